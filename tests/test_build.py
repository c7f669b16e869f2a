"""Host-side checks of the in-tree build script (CPU only: hipcc cross-compiles
for gfx950 without a GPU)."""
import os

import pytest

import indexer_top_sparse_02_amd.build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")


def test_indexer_sources_take_the_placement_switches():
    flags = B.FILE_FLAGS["indexer.hip"]
    assert B._NO_SINK[1] in flags and "-amdgpu-mfma-vgpr-form" in flags
    # every -mllvm is followed by its option
    for i, f in enumerate(flags):
        if f == "-mllvm":
            assert i + 1 < len(flags) and flags[i + 1].startswith("-")


def test_compile_falls_back_where_the_compiler_lacks_the_sinking_switch(tmp_path, monkeypatch, capsys):
    src = tmp_path / "tiny.hip"
    src.write_text("#include <hip/hip_runtime.h>\n__global__ void k(float* x) { x[threadIdx.x] += 1.f; }\n")
    bogus = ["-mllvm", "-no-such-sinking-switch"]
    monkeypatch.setattr(B, "BUILD", str(tmp_path / "build"))
    monkeypatch.setattr(B, "_NO_SINK", bogus)
    monkeypatch.setitem(B.FILE_FLAGS, "tiny.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"] + bogus)
    os.makedirs(B.BUILD, exist_ok=True)
    obj = B._compile(str(src))
    assert os.path.getsize(obj) > 0
    assert "building without it" in capsys.readouterr().err


def test_compile_still_reports_other_errors(tmp_path, monkeypatch):
    src = tmp_path / "broken.hip"
    src.write_text("this is not C++\n")
    monkeypatch.setattr(B, "BUILD", str(tmp_path / "build"))
    os.makedirs(B.BUILD, exist_ok=True)
    with pytest.raises(RuntimeError, match="hipcc failed"):
        B._compile(str(src))
