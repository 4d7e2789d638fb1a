"""Host-side checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments with the documented status codes before
anything reaches a GPU.  Runs without a GPU."""
import ctypes
import os

import pytest
import torch

import qwen2_decoder_forward_amd as q2
from qwen2_decoder_forward_amd import _lib


def test_library_exports_every_header_function():
    names = q2.header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(q2.lib, n), f"{n} declared in q2.h but not exported"
        assert n in _lib._SIGS, f"{n} has no ctypes signature"
    assert q2.version().startswith("q2")


def test_descriptor_layout_matches_header(tmp_path):
    """The ctypes structures have the sizes and field offsets the C compiler
    gives the header's structs."""
    src = tmp_path / "layout.c"
    fields = {"q2_tensor": [f for f, _ in _lib.Q2Tensor._fields_],
              "q2_config": [f for f, _ in _lib.Q2Config._fields_]}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "q2.h"', "int main(void) {"]
    for st, fs in fields.items():
        lines.append(f'printf("%zu\\n", sizeof({st}));')
        lines += [f'printf("%zu\\n", offsetof({st}, {f}));' for f in fs]
    lines += ["return 0;", "}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = []
    for cls in (_lib.Q2Tensor, _lib.Q2Config):
        want.append(ctypes.sizeof(cls))
        want += [getattr(cls, f).offset for f, _ in cls._fields_]
    assert got == want


def _err(fn, *args):
    with pytest.raises(q2.Q2Error) as e:
        fn(*args)
    return e.value.name


def test_validation_errors_without_gpu():
    bf = torch.bfloat16
    x = torch.zeros(4, 64, dtype=bf)
    w = torch.zeros(32, 64, dtype=bf)
    out = torch.zeros(4, 32, dtype=bf)
    # shape mismatch
    assert _err(q2.q2_linear, torch.zeros(4, 31, dtype=bf), x, w) == "Q2_ESHAPE"
    assert _err(q2.q2_linear, out, torch.zeros(4, 63, dtype=bf), w) == "Q2_ESHAPE"
    # dtype mismatch
    assert _err(q2.q2_linear, out, x.float(), w) == "Q2_EDTYPE"
    # non-contiguous last dim
    assert _err(q2.q2_linear, out, torch.zeros(64, 4, dtype=bf).t(), w) == "Q2_ESTRIDE"
    # bias of the wrong length
    assert _err(q2.q2_linear, out, x, w, torch.zeros(31, dtype=bf)) == "Q2_ESHAPE"
    # rms_norm weight size
    assert _err(q2.q2_rms_norm, x, x, torch.zeros(63, dtype=bf), 1e-6) == "Q2_ESHAPE"
    assert _err(q2.q2_rms_norm, x, x, torch.zeros(64, dtype=bf), -1.0) == "Q2_EINVAL"
    # rope: odd head dim, wrong pos dtype
    assert _err(q2.q2_rope, torch.zeros(2, 3, 5), torch.zeros(2, 3, 5), torch.zeros(2, dtype=torch.int64),
                1e4) == "Q2_ESHAPE"
    assert _err(q2.q2_rope, torch.zeros(2, 3, 4), torch.zeros(2, 3, 4), torch.zeros(2), 1e4) == "Q2_EDTYPE"
    # attention: nh not a multiple of nkv, S < T, unsupported bf16 head dim
    q = torch.zeros(4, 6, 128, dtype=bf)
    assert _err(q2.q2_self_attention, q, q, torch.zeros(4, 4, 128, dtype=bf), torch.zeros(4, 4, 128, dtype=bf),
                0.1) == "Q2_ESHAPE"
    assert _err(q2.q2_self_attention, q, q, torch.zeros(3, 2, 128, dtype=bf), torch.zeros(3, 2, 128, dtype=bf),
                0.1) == "Q2_ESHAPE"
    q64 = torch.zeros(4, 6, 64, dtype=bf)
    assert _err(q2.q2_self_attention, q64, q64, torch.zeros(4, 2, 64, dtype=bf), torch.zeros(4, 2, 64, dtype=bf),
                0.1) == "Q2_ESHAPE"
    # swiglu/add shape and dtype mismatch
    assert _err(q2.q2_add, x, x, torch.zeros(4, 65, dtype=bf)) == "Q2_ESHAPE"
    assert _err(q2.q2_swiglu, x, x, x.float()) == "Q2_EDTYPE"
    # argmax: wrong index dtype / count
    v = torch.zeros(3, 100)
    with pytest.raises(TypeError):
        q2.q2_argmax(torch.zeros(3, dtype=torch.int32), torch.zeros(3), v)
    assert _err(q2.q2_argmax, torch.zeros(3), torch.zeros(3), v) == "Q2_EDTYPE"
    assert _err(q2.q2_argmax, torch.zeros(2, dtype=torch.int64), torch.zeros(2), v) == "Q2_ESHAPE"
    # embedding: ids must be int64, hidden sizes must agree
    assert _err(q2.q2_embedding, torch.zeros(3, 8), torch.zeros(3), torch.zeros(10, 8)) == "Q2_EDTYPE"
    assert _err(q2.q2_embedding, torch.zeros(3, 8), torch.zeros(3, dtype=torch.int64),
                torch.zeros(10, 9)) == "Q2_ESHAPE"
    # rearrange: shape / dtype mismatch
    assert _err(q2.q2_rearrange, torch.zeros(2, 3), torch.zeros(3, 2)) == "Q2_ESHAPE"
    assert _err(q2.q2_rearrange, torch.zeros(2, 3), torch.zeros(2, 3, dtype=bf)) == "Q2_EDTYPE"


def test_model_config_validation_without_gpu():
    from qwen2_decoder_forward_amd.model import make_config
    import synth
    sh = synth.SHAPES["1.5b"]
    bad = make_config(sh, 128, 1)
    bad.nkv = 5                        # 12 heads not a multiple of 5
    assert _err(q2.q2_model_create, bad) == "Q2_ESHAPE"
    bad = make_config(sh, 128, 65)     # batch above the supported 64
    assert _err(q2.q2_model_create, bad) == "Q2_ESHAPE"
    bad = make_config(sh, 128, 1)
    bad.dtype = 2
    assert _err(q2.q2_model_create, bad) == "Q2_EDTYPE"
    bad = make_config(sh, 0, 1)
    assert _err(q2.q2_model_create, bad) == "Q2_ESHAPE"


def test_valid_model_without_gpu_is_an_error_not_a_crash():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from qwen2_decoder_forward_amd.model import make_config
    import synth
    cfg = make_config(synth.SHAPES["tiny"], 32, 1)
    assert _err(q2.q2_model_create, cfg) in ("Q2_EINVAL", "Q2_EHIP")


def test_decode_attention_split_plan_without_gpu():
    """The split-KV plan of the decode attention, seen through the workspace
    it asks for (float32 partials [B * nkv][splits][16][128] plus a (max, sum)
    pair per row): keys in chunks of whole 64-key blocks, at most two
    workgroups per CU (512), and at most 8 splits once 8 already give every
    CU a workgroup (B * nkv >= 32)."""
    per_split = 16 * (128 * 4 + 8)

    def splits(B, S, nh, nkv):
        return q2.q2_self_attention_workspace_bytes(B, 1, S, nh, nkv, 128) // (B * nkv * per_split)

    assert splits(1, 192, 12, 2) == 3      # batch-1 decode at its last step: 3 x 64 keys
    assert splits(64, 4097, 12, 2) == 4    # 64 x 4097: 128 (sequence, KV head) pairs, 4 splits each
    assert splits(8, 1280, 28, 4) == 7     # 7B batch 8: capped at 8 -> 7 x 192 keys
    assert splits(4, 800, 28, 4) == 13     # 16 pairs: 13 x 64 keys (8 would leave CUs idle)
    assert q2.q2_self_attention_workspace_bytes(1, 1, 64, 12, 2, 128) == 0   # one split, no partials
