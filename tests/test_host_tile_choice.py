"""The expert-GEMM kernel choices at the workload shapes, checked on the host:
a small program compiled against the library's ffn.hip prints the row tile
of each GEMM (16/32/64: direct kernel, 128/256: LDS-tiled) and whether the
shared expert's GEMMs ride in the routed launches.  The expected values are
the measured choices the kernel sources document."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_amd", "csrc")


@pytest.fixture(scope="module")
def tile_choice(tmp_path_factory):
    from mixture_experts_layer_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("host") / "tile_choice")
    cmd = [hipcc, "-O1", "-std=c++17", f"--offload-arch={B.ARCH}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "tile_choice.cpp"), os.path.join(CSRC, "ffn.hip"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]

    def run(H, I, Is, E, E_loc, k, T):
        out = subprocess.run([exe] + [str(v) for v in (H, I, Is, E, E_loc, k, T)],
                             capture_output=True, text=True, check=True).stdout.split()
        return dict(zip(out[0::2], out[1::2]))
    return run


# (shape, T) -> expected choices
CASES = [
    # Qwen3 EP view: direct at a few rows, 128-row LDS tiles from 64 rows per
    # expert, 256-row tiles at prefill
    (("qwen3_ep", 4096, 1536, 0, 128, 128, 8, 16), dict(gate_up="16", down="16")),
    (("qwen3_ep", 4096, 1536, 0, 128, 128, 8, 1024),
     dict(gate_up="128", down="128", down_cols="256")),
    (("qwen3_ep", 4096, 1536, 0, 128, 128, 8, 8192), dict(gate_up="256", down="256")),
    # Qwen3 TP share (I/P = 192): direct kernel at T <= 64; 8-column gate/up
    # tiles while 16-column ones would give fewer than 3 blocks per CU
    # (T = 8: about 50 touched experts x 12 column tiles)
    (("qwen3_tp", 4096, 192, 0, 128, 128, 8, 4), dict(gate_up="16", gate_up_cols="8")),
    (("qwen3_tp", 4096, 192, 0, 128, 128, 8, 8), dict(gate_up="16", gate_up_cols="8")),
    (("qwen3_tp", 4096, 192, 0, 128, 128, 8, 16), dict(gate_up="16", gate_up_cols="16")),
    (("qwen3_tp", 4096, 192, 0, 128, 128, 8, 64),
     dict(gate_up="16", down="16", gate_up_cols="16")),
    # EP view T = 1: 8 experts x 96 tiles, 3 per CU (expected 7.8 experts:
    # narrowed; measured 1% faster narrowed), T = 16: 30 per CU
    (("qwen3_ep", 4096, 1536, 0, 128, 128, 8, 1), dict(gate_up="16", gate_up_cols="8")),
    (("qwen3_ep", 4096, 1536, 0, 128, 128, 8, 16), dict(gate_up="16", gate_up_cols="16")),
    # Mixtral: direct at T = 16, 256-row tiles at 4096; at T = 64-256 (one
    # 128-row tile per expert) the down projection takes 128-column tiles so
    # that its blocks fill the CUs, at T = 512 (a second tile for many
    # experts) no longer
    (("mixtral", 4096, 14336, 0, 8, 8, 2, 16), dict(gate_up="16", down="16")),
    (("mixtral", 4096, 14336, 0, 8, 8, 2, 64), dict(gate_up="128", down="128", down_cols="128")),
    (("mixtral", 4096, 14336, 0, 8, 8, 2, 256), dict(gate_up="128", down="128", down_cols="128")),
    (("mixtral", 4096, 14336, 0, 8, 8, 2, 512), dict(gate_up="128", down="128", down_cols="256")),
    (("mixtral", 4096, 14336, 0, 8, 8, 2, 4096), dict(gate_up="256", down="256", down_cols="256")),
    # DeepSeek-V3: direct at T = 1 (shared expert in both routed launches);
    # at T = 8 and 16 the gate/up GEMM on LDS tiles, the down projection
    # direct walking its map, the shared expert riding in both (switched to
    # the routed tile: its gate/up at T = 8, its down projection at T = 16,
    # where its own tile already is the routed gate/up one); at T = 64 all
    # on LDS tiles; at 4096 the shared expert in launches of its own
    (("deepseek", 7168, 2048, 2048, 256, 256, 8, 1),
     dict(gate_up="16", down="16", shared_gate_up="shared", shared_down="shared")),
    (("deepseek", 7168, 2048, 2048, 256, 256, 8, 8),
     dict(gate_up="128", down="16", shared_gate_up="shared_switched", shared_down="shared")),
    (("deepseek", 7168, 2048, 2048, 256, 256, 8, 16),
     dict(gate_up="128", down="16", shared_gate_up="shared", shared_down="shared_switched")),
    (("deepseek", 7168, 2048, 2048, 256, 256, 8, 64),
     dict(gate_up="128", down="128", shared_gate_up="shared", shared_down="shared")),
    (("deepseek", 7168, 2048, 2048, 256, 256, 8, 4096),
     dict(gate_up="128", down="128", shared_gate_up="own", shared_down="own")),
    # the shapes of the GPU test of the shared expert's launches
    # (test_gpu_parity.py), one per combination of the two choices
    (("small_shared", 1024, 256, 256, 64, 64, 8, 1),
     dict(gate_up="16", shared_gate_up="shared", shared_down="shared")),
    (("small_shared", 1024, 256, 256, 64, 64, 8, 16),
     dict(gate_up="16", shared_gate_up="shared_switched", shared_down="shared_switched")),
    (("small_shared", 1024, 256, 256, 64, 64, 8, 64),
     dict(gate_up="128", shared_gate_up="shared", shared_down="shared")),
    (("small_shared", 1024, 256, 256, 64, 64, 8, 600),
     dict(gate_up="128", shared_expert="256", shared_gate_up="shared_switched",
          shared_down="shared_switched")),
    # (both down projections in the kernel that shares its rows' activations
    # through LDS, which any two can share a launch of)
    (("small_shared", 1024, 256, 512, 64, 64, 8, 1),
     dict(gate_up="16", shared_gate_up="shared", shared_down="shared")),
    (("small_shared", 1024, 256, 512, 64, 64, 8, 16),
     dict(gate_up="16", shared_gate_up="shared_switched", shared_down="shared_switched",
          shared_down_tile="16")),
    # a 4096-long shared down contraction is past that kernel's LDS, and its
    # direct kernel takes more waves per block than the routed one: the
    # shared gate/up GEMM rides in the routed launch, its down projection
    # has its own
    (("wide_shared_down", 1024, 256, 4096, 64, 64, 8, 1),
     dict(gate_up="16", shared_gate_up="shared", shared_down="own")),
    (("wide_shared_down", 1024, 256, 4096, 64, 64, 8, 16),
     dict(gate_up="16", shared_gate_up="shared_switched", shared_down="own",
          shared_down_tile="128")),
    (("small_shared", 1024, 256, 512, 64, 64, 8, 64),
     dict(gate_up="128", shared_gate_up="shared", shared_down="shared")),
    (("wide_shared", 6144, 2048, 4096, 32, 32, 8, 4),
     dict(gate_up="128", down="16", shared_gate_up="own", shared_down="shared")),
    # 256-row tiles on both problems: the shared expert's 1636 dense rows end
    # in a 100-row tile inside the routed launches (the GPU test of this shape
    # checks its wide half tile)
    (("big_shared", 512, 256, 256, 32, 32, 8, 1636),
     dict(gate_up="256", down="256", shared_gate_up="shared", shared_down="shared",
          shared_gate_up_tile="256", shared_down_tile="256")),
]


@pytest.mark.parametrize("case,want", CASES, ids=[f"{c[0]}-T{c[-1]}" for c, _ in CASES])
def test_tile_choice(tile_choice, case, want):
    got = tile_choice(*case[1:])
    for key, value in want.items():
        assert got[key] == value, (key, got)
