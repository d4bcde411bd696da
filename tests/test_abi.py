"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/afd_ffn.h declares,
agree with a C compiler on the struct layouts, and reject bad arguments
synchronously with the documented status codes before touching the device.
"""
import ctypes
import os
import subprocess

import pytest

from expert_side_attention_amd import _ffi as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.LIB_PATH):
        from expert_side_attention_amd import build
        build.build()
    return F.load_library()


def test_exports_every_header_function(lib):
    names = F.header_functions()
    assert len(names) >= 9
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_struct_layout_matches_c_compiler(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "afd_ffn.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(afd_ffn_config),
         sizeof(afd_ffn_weights), sizeof(afd_ffn_trace),
         offsetof(afd_ffn_config, max_tokens), offsetof(afd_ffn_weights, down_s),
         offsetof(afd_ffn_weights, sh_down_s), offsetof(afd_ffn_trace, x_s),
         offsetof(afd_ffn_trace, num_tiles), offsetof(afd_ffn_config, split_gemms),
         offsetof(afd_ffn_trace, sync_timeouts));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I",
                    os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                       check=True).stdout.split()))
    want = [ctypes.sizeof(F.afd_ffn_config), ctypes.sizeof(F.afd_ffn_weights),
            ctypes.sizeof(F.afd_ffn_trace), F.afd_ffn_config.max_tokens.offset,
            F.afd_ffn_weights.down_s.offset, F.afd_ffn_weights.sh_down_s.offset,
            F.afd_ffn_trace.x_s.offset, F.afd_ffn_trace.num_tiles.offset,
            F.afd_ffn_config.split_gemms.offset, F.afd_ffn_trace.sync_timeouts.offset]
    assert got == want


def _cfg(**kw):
    base = dict(abi_version=F.AFD_FFN_ABI_VERSION, mode=F.AFD_MODE_BF16, hidden=256,
                num_experts=8, top_k=2, inter=512, num_shared=0, shared_inter=0,
                max_tokens=16, has_router_bias=0)
    base.update(kw)
    return F.afd_ffn_config(**base)


def _w(**kw):
    fake = 0x1000  # never dereferenced: validation fails before any use
    base = dict(router_w=fake, gate_w=fake, up_w=fake, down_w=fake)
    base.update(kw)
    return F.afd_ffn_weights(**base)


@pytest.mark.parametrize("cfg,w,status,needle", [
    (dict(abi_version=99), {}, F.AFD_ERR_INVALID_ARG, "abi_version"),
    (dict(mode=7), {}, F.AFD_ERR_INVALID_ARG, "mode"),
    (dict(num_experts=0), {}, F.AFD_ERR_INVALID_ARG, "num_experts"),
    (dict(num_experts=1024), {}, F.AFD_ERR_UNSUPPORTED, "num_experts"),
    (dict(top_k=0), {}, F.AFD_ERR_INVALID_ARG, "top_k"),
    (dict(top_k=9), {}, F.AFD_ERR_INVALID_ARG, "top_k"),
    (dict(hidden=200), {}, F.AFD_ERR_INVALID_ARG, "hidden"),
    (dict(inter=0), {}, F.AFD_ERR_INVALID_ARG, "inter"),
    (dict(num_shared=1, shared_inter=100), {}, F.AFD_ERR_INVALID_ARG, "shared_inter"),
    (dict(num_shared=-1), {}, F.AFD_ERR_INVALID_ARG, "num_shared"),
    (dict(max_tokens=0), {}, F.AFD_ERR_INVALID_ARG, "max_tokens"),
    (dict(has_router_bias=1), {}, F.AFD_ERR_INVALID_ARG, "router_b"),
    (dict(single_launch=2), {}, F.AFD_ERR_INVALID_ARG, "single_launch"),
    (dict(split_gemms=-1), {}, F.AFD_ERR_INVALID_ARG, "split_gemms"),
    ({}, dict(gate_w=None), F.AFD_ERR_INVALID_ARG, "gate_w"),
    (dict(mode=F.AFD_MODE_W8A8_E4M3), {}, F.AFD_ERR_INVALID_ARG, "gate_s"),
    (dict(num_shared=1, shared_inter=256), {}, F.AFD_ERR_INVALID_ARG, "sh_gate_w"),
    ({}, dict(up_w=0x1008), F.AFD_ERR_INVALID_ARG, "16-byte aligned"),
    (dict(has_router_bias=1), dict(router_b=0x1002), F.AFD_ERR_INVALID_ARG, "4-byte aligned"),
])
def test_create_rejects_bad_config(lib, cfg, w, status, needle):
    with pytest.raises(F.AfdError) as ei:
        F.afd_ffn_create(_cfg(**cfg), _w(**w))
    assert ei.value.status == status
    assert needle in F.afd_ffn_last_error()


def test_null_arguments_rejected(lib):
    h = ctypes.c_void_p()
    assert lib.afd_ffn_create(None, ctypes.byref(_w()), ctypes.byref(h)) == F.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_create(ctypes.byref(_cfg()), None, ctypes.byref(h)) == F.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_create(ctypes.byref(_cfg()), ctypes.byref(_w()), None) == F.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_forward(None, 1, 2, 4, None) == F.AFD_ERR_INVALID_ARG
    tr = F.afd_ffn_trace()
    assert lib.afd_ffn_forward_traced(None, 1, 2, 4, None, ctypes.byref(tr)) == F.AFD_ERR_INVALID_ARG
    assert lib.afd_quant_fp8_1x128(None, 4, 128, 1, 2, None) == F.AFD_ERR_INVALID_ARG
    assert lib.afd_quant_fp8_1x128(1, 4, 100, 1, 2, None) == F.AFD_ERR_INVALID_ARG
    assert lib.afd_quant_fp8_128x128(1, 100, 128, 1, 2, None) == F.AFD_ERR_INVALID_ARG
    # misaligned buffers are refused before anything is launched
    assert lib.afd_quant_fp8_1x128(0x1008, 4, 128, 0x2000, 0x3000, None) == F.AFD_ERR_INVALID_ARG
    assert "aligned" in F.afd_ffn_last_error()
    assert lib.afd_quant_fp8_1x128_f32(0x1000, 4, 128, 0x2000, 0x3002, None) == F.AFD_ERR_INVALID_ARG
    assert lib.afd_quant_fp8_128x128(0x1000, 128, 128, 0x2004, 0x3000, None) == F.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_profile_enable(None, 1) == F.AFD_ERR_INVALID_ARG
    lib.afd_ffn_destroy(None)  # ignored
