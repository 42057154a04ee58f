"""The library's kernels, compiled for gfx950 with the flags build() uses, never touch a register
that an LDS read still has to write (tests/isa_lds.py), on any path through the kernel; and the
scan itself catches such a use, planted in a small assembly listing."""
import os
import shutil
import subprocess

import pytest

import isa_lds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

LISTING = """\
_ZN4demo1kEv:
\tds_read_b128 v[4:7], v1 offset:16
\tv_add_f32 v8, v9, v10
\ts_waitcnt lgkmcnt(0)
\tv_add_f32 v8, v4, v10
.LBB0_1:
\tds_read_b32 v2, v1
\tds_read_b32 v3, v1 offset:4
\ts_waitcnt lgkmcnt(1)
\tv_mov_b32 v11, v2
\ts_waitcnt lgkmcnt(0)
\tv_mov_b32 v12, v3
\tds_read_b32 v13, v1 offset:8
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
.Lfunc_end0:
"""


def test_scan_is_clean_on_a_correct_listing():
    assert isa_lds.hazards(LISTING, "_ZN4demo1kEv") == []


@pytest.mark.parametrize("bad,planted", [
    # a use of a read's register before any wait
    ("\tv_add_f32 v8, v9, v10\n", "\tv_add_f32 v8, v5, v10\n"),
    # a wait that leaves the read in flight (lgkmcnt(1) covers only the older of two reads)
    ("\tv_mov_b32 v11, v2\n", "\tv_mov_b32 v11, v3\n"),
    # a use at the top of a loop of a read issued at its bottom (back-edge)
    ("\tds_read_b32 v2, v1\n", "\tv_mov_b32 v14, v13\n\tds_read_b32 v2, v1\n"),
    # an overwrite of a register still in flight
    ("\tv_add_f32 v8, v9, v10\n", "\tv_add_f32 v6, v9, v10\n"),
])
def test_scan_catches_a_planted_use(bad, planted):
    listing = LISTING.replace(bad, planted, 1)
    assert listing != LISTING
    assert isa_lds.hazards(listing, "_ZN4demo1kEv")


def test_library_kernels_wait_for_their_lds_reads(tmp_path):
    import __graft_entry__ as entry
    hipcc = entry.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    flags = [f for f in entry.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / "q6k.s"
    subprocess.check_call([hipcc] + flags + ["-S", "--cuda-device-only",
                                             os.path.join(ROOT, "q6_int8_prefill_amd", "csrc",
                                                          "q6k.hip"), "-o", str(out)],
                          stderr=subprocess.DEVNULL)
    asm = out.read_text()
    names = isa_lds.kernel_names(asm)
    gemms = [n for n in names if any(k in n for k in ("gemm_kernel", "folded_kernel"))]
    assert len(gemms) == 8  # layouts 0, 1, 2 and q4_K, each with its dots export
    checked = [n for n in names if "kernel" in n]
    for name in checked:
        found = isa_lds.hazards(asm, name)
        assert not found, (name, found[:5])
