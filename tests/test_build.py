"""The build script's check of the M0 invariant that the loads into LDS rely on: the loads
set M0 inside their own inline-assembly block, which is sound only while nothing the
compiler emits keeps a value in M0 (the compiler does not honour M0 in a clobber list)."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("fa_build", os.path.join(ROOT, "exact_block_sparse_amd", "build.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


GOOD = """\
\t;;#ASMSTART
\ts_mov_b32 m0, s24
\tbuffer_load_dwordx4 v198, s[16:19], 0 offen lds
\t;;#ASMEND
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]
"""


def test_check_m0_accepts_the_kernels_pattern():
    assert _build_module().check_m0(GOOD) == []


@pytest.mark.parametrize("bad", [
    "\ts_mov_b32 m0, -1\n" + GOOD,                                  # the compiler sets M0 itself
    GOOD + "\tv_readlane_b32 s0, v1, m0\n",                         # ... or reads it
    "\t;;#ASMSTART\n\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds\n\t;;#ASMEND\n",   # no M0 move
    "\tbuffer_load_dword v1, s[0:3], 0 offen lds\n",                # a load into LDS the compiler placed
    GOOD + "\tv_movrels_b32 v0, v1\n",                              # implicit M0 use
    GOOD + "\ts_sendmsg sendmsg(MSG_DEALLOC_VGPRS)\n",
])
def test_check_m0_rejects_other_uses(bad):
    assert _build_module().check_m0(bad)


@pytest.mark.parametrize("src", ["fa_fwd.hip", "fa_bwd.hip"])
def test_built_kernels_keep_the_m0_invariant(src):
    path = os.path.join(ROOT, "_build", src + ".s")
    if not os.path.exists(path):
        pytest.skip("library not built in this tree")
    text = open(path).read()
    assert "buffer_load_dwordx4" in text and " lds" in text
    assert _build_module().check_m0(text) == []
