"""The C-ABI library loads on the host and exports every function include/specdec.h declares."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specdec.h")
LIB = os.path.join(ROOT, "block_verify_amd", "libspecdec.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(specdec_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_path_calls():
    names = _declared()
    for n in ("specdec_prefill", "specdec_decode_step", "specdec_verify_round", "specdec_kv_trim"):
        assert n in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_binding_covers_every_declared_symbol():
    from block_verify_amd import lib as binding
    assert sorted(binding.EXPORTED) == _declared()


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_host_validation_without_gpu():
    """Argument checks that need no device: sizes, bad shapes, status strings."""
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import QWEN_1_5B, TINY
    L = b.lib()
    d = b.desc_of(QWEN_1_5B)
    n = ctypes.c_size_t()
    assert L.specdec_weights_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value >= QWEN_1_5B.weight_bytes_bf16()
    assert L.specdec_tensor_count(ctypes.byref(d)) == len(QWEN_1_5B.tensor_specs())
    assert L.specdec_workspace_bytes(ctypes.byref(d), 33, 4096, ctypes.byref(n)) == b.ECAPACITY
    bad = b.desc_of(TINY)
    bad.head_dim = 96
    assert L.specdec_weights_bytes(ctypes.byref(bad), ctypes.byref(n)) == b.ESHAPE
    bad = b.desc_of(TINY)
    bad.n_q_heads = 3
    assert L.specdec_weights_bytes(ctypes.byref(bad), ctypes.byref(n)) == b.ESHAPE
    bad = b.desc_of(TINY)
    bad.hidden = 4096 + 32   # the norm scale reads at most 256 partials of 16 features
    assert L.specdec_weights_bytes(ctypes.byref(bad), ctypes.byref(n)) == b.ESHAPE
    assert L.specdec_cache_bytes(ctypes.byref(b.desc_of(TINY)), 0, ctypes.byref(n)) == b.EINVAL
    assert L.specdec_decode_step(None, None, None, 1, None, None, None, None, 0, None) == b.EINVAL
    assert L.specdec_round_create(None, None) == b.EINVAL
    assert L.specdec_status_str(b.EDEVICE) == b"device error flag set"
    assert L.specdec_round_state_bytes(64, ctypes.byref(n)) == 0 and n.value == 64 + 64 * 4


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_q4_blob_size_and_shape_checks():
    """4-bit models: blob = 0.5 byte codes + 8 bytes of (scale, zero) per 128 inputs per row,
    plus the bf16 embedding / LM head and fp32 gains; unsupported shapes are refused."""
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import QWEN_7B, TINY
    L = b.lib()
    n = ctypes.c_size_t()
    d = b.desc_of(QWEN_7B, b.W_Q4G64)
    assert L.specdec_weights_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    S = QWEN_7B
    lin = 0
    for rows, k in [((S.n_q_heads + 2 * S.n_kv_heads) * S.head_dim, S.hidden), (S.hidden, S.n_q_heads * S.head_dim),
                    (2 * S.ffn, S.hidden), (S.hidden, S.ffn)]:
        nb = -(-k // 128)
        lin += rows * nb * 64 + rows * nb * 8
    bf16 = 2 * S.vocab * S.hidden * 2
    assert n.value >= S.n_layers * lin + bf16
    assert n.value < S.n_layers * lin + bf16 + 4 * 1024 * 1024   # alignment and gains only
    bad = b.desc_of(TINY, b.W_Q4G64)
    bad.ffn = 1056   # a multiple of 32, not of 64
    assert L.specdec_weights_bytes(ctypes.byref(bad), ctypes.byref(n)) == b.ESHAPE
    big = b.desc_of(TINY, b.W_Q4G64)
    big.hidden = 8192   # past the hidden limit (and the 4-bit kernel's LDS budget)
    assert L.specdec_weights_bytes(ctypes.byref(big), ctypes.byref(n)) == b.ESHAPE


def test_binding_structs_match_the_header_layout(tmp_path):
    """Every field of the ctypes mirrors sits at the offset the C compiler gives it in
    include/specdec.h (gcc on the host), and the structs have the same size."""
    import shutil
    import subprocess
    from block_verify_amd import lib as b
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    structs = {"specdec_round_desc": b.RoundDesc, "specdec_model_desc": b.ModelDesc,
               "specdec_round_state": b.RoundState}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    for line in filter(None, out):
        cname, fname, val = line.split()
        py = structs[cname]
        got = ctypes.sizeof(py) if fname == "sizeof" else getattr(py, fname).offset
        assert got == int(val), (cname, fname, got, val)
