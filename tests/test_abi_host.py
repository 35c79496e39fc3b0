"""Host-side checks of the C ABI (no GPU needed, no kernel is launched):
every symbol include/pa.h declares is exported, and every argument error is
reported before anything is enqueued."""
import ctypes
import os
import re

import pytest

import paged_kv_decode_pa_amd as pa
from paged_kv_decode_pa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert pa.status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert pa.status_string(code) not in ("ok", "unknown status")
    assert pa.status_string(-99) == "unknown status"


def test_workspace_size_arithmetic():
    # plan: order [B] int32, a 256-byte item count, items [B * NP] int32
    # pairs (each padded to 256 B); then, when split, [B, Hq, NP, D] fp32 +
    # two [B, Hq, NP] fp32
    def pad(n):
        return (n + 255) // 256 * 256

    def plan(B, NP):
        return pad(B * 4) + 256 + pad(B * NP * 8)
    B, Hq, D, L, P = 33, 32, 64, 131072, 512
    NP = L // P
    assert pa.workspace_size(B, Hq, D, L, P) == plan(B, NP) + B * Hq * NP * (D + 2) * 4
    assert pa.workspace_size(B, Hq, D, L, 0) == plan(B, 1)         # no split
    assert pa.workspace_size(B, Hq, D, 300, 512) == plan(B, 1)     # one partition
    assert pa.workspace_size(4, 8, 256, 513, 512) == plan(4, 2) + 4 * 8 * 2 * 258 * 4
    assert pa.workspace_size(0, 8, 256, 513, 512) == 0


def test_partition_choice_is_a_multiple_of_block_size():
    for bs in (1, 16, 32):
        for B, L in ((512, 1024), (16, 8192), (33, 131072), (4, 255)):
            P = pa.partition_size(B, 8, 4, 256, bs, L)
            assert P >= 0 and P % bs == 0


def test_partition_choice_splits_only_long_or_few():
    # enough (sequence, KV head) units for short contexts: one partition
    assert pa.partition_size(64, 8, 4, 256, 16, 1024) == 0
    assert pa.partition_size(512, 8, 4, 256, 16, 2048) == 0
    # long contexts or few units: 512-token partitions
    assert pa.partition_size(16, 8, 4, 256, 16, 8192) == 512
    assert pa.partition_size(8, 8, 4, 256, 16, 1024) == 512
    assert pa.partition_size(33, 32, 4, 64, 32, 131072) == 512


def decode_args(**over):
    a = dict(out=FAKE, ws=None, ws_bytes=0, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, maxb=8,
             cl=FAKE, maxL=128, B=2, Hq=8, Hkv=2, D=64, bs=16, NB=64, scale=0.125,
             softcap=0.0, window=0, P=0, dt=_lib.PA_F32, stream=None)
    a.update(over)
    return a


def call_decode(a):
    lib = _lib.load()
    return lib.pa_decode(a["out"], a["ws"], a["ws_bytes"], a["q"], a["kc"], a["vc"], a["bt"],
                         a["maxb"], a["cl"], a["maxL"], a["B"], a["Hq"], a["Hkv"], a["D"],
                         a["bs"], a["NB"], a["scale"], a["softcap"], a["window"], a["P"],
                         a["dt"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(out=None), -1),
    (dict(q=None), -1),
    (dict(kc=None), -1),
    (dict(bt=None), -1),
    (dict(cl=None), -1),
    (dict(Hq=6, Hkv=4), -1),              # heads not a multiple of kv heads
    (dict(B=-1), -1),
    (dict(maxL=129), -1),                 # more than max_blocks * block_size
    (dict(P=24), -1),                     # not a multiple of block_size
    (dict(P=-16), -1),
    (dict(window=-1), -1),
    (dict(softcap=-1.0), -1),
    (dict(scale=float("nan")), -1),
    (dict(D=96), -2),
    (dict(dt=7), -2),
    (dict(bs=12), -2),
    (dict(Hq=32, Hkv=2), -2),             # group of 16 not built
    (dict(Hq=6, Hkv=2), -2),              # group of 3 not built
    (dict(P=16, maxL=128), -3),           # no workspace
    (dict(P=0, maxL=128), -3),            # the work order needs one too
    (dict(P=16, maxL=128, ws=FAKE, ws_bytes=300), -3),
])
def test_decode_rejects_bad_arguments(over, status):
    assert call_decode(decode_args(**over)) == status


def test_decode_with_no_sequences_is_a_noop():
    assert call_decode(decode_args(B=0, out=None, q=None)) == 0


def test_reduce_argument_checks():
    lib = _lib.load()
    # no split: nothing to reduce, nothing touched
    assert lib.pa_decode_reduce(None, None, 0, None, 128, 2, 8, 64, 0, 0, 0, None) == 0
    assert lib.pa_decode_reduce(FAKE, None, 0, FAKE, 128, 2, 8, 64, 16, 0, 0, None) == -3
    assert lib.pa_decode_reduce(FAKE, FAKE, 10, FAKE, 128, 2, 8, 64, 16, 0, 0, None) == -3
    assert lib.pa_decode_reduce(FAKE, FAKE, 1 << 20, FAKE, 128, 2, 8, 96, 16, 0, 0, None) == -2
    assert lib.pa_decode_reduce(FAKE, FAKE, 1 << 20, FAKE, 128, 2, 8, 64, -1, 0, 0, None) == -1


def test_reshape_argument_checks():
    lib = _lib.load()
    f = lib.pa_reshape_and_cache
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 16, 2, 64, 0, None) == 0   # no tokens
    assert f(None, FAKE, FAKE, FAKE, FAKE, 4, 64, 16, 2, 64, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, 64, 16, 2, 64, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 64, 16, 2, 64, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 16, 2, 80, 0, None) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 3, 2, 64, 0, None) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 16, 2, 64, 5, None) == -2


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError):
        pa.decode(q, torch.zeros(4, 16, 1, 64), torch.zeros(4, 16, 1, 64),
                  torch.zeros(1, 1, dtype=torch.int32), torch.ones(1, dtype=torch.int32),
                  0.125, max_context_len=1, partition_size=0)


@pytest.mark.parametrize("mirror,cname", [(_lib.StepArgs, "pa_step_args"),
                                          (_lib.MQStepArgs, "pa_mq_step_args")])
def test_step_args_layout_matches_the_header(tmp_path, mirror, cname):
    """The ctypes mirrors of pa_step_args and pa_mq_step_args have the C
    structs' sizes and offsets (checked with the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = [f for f, _ in mirror._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"pa.h\"\n"
        f"int main(void) {{ printf(\"%zu\\n\", sizeof({cname}));\n"
        + "".join(f'  printf("%zu\\n", offsetof({cname}, {f}));\n' for f in fields)
        + "  return 0; }\n")
    exe = tmp_path / "layout"
    # pa.h only needs the standard headers for this; hipStream_t is void*
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(mirror)
    for f, off in zip(fields, got[1:]):
        assert getattr(mirror, f).offset == off, f


def test_step_graph_argument_checks():
    lib = _lib.load()
    assert lib.pa_step(None, None) == -1
    h = ctypes.c_void_p()
    assert lib.pa_step_graph_create(None, None, ctypes.byref(h)) == -1
    assert lib.pa_step_graph_launch(None, None) == -1
    assert lib.pa_step_graph_destroy(None) == 0


# --------------------------------------------------------------------------
# multi-query attention
# --------------------------------------------------------------------------
def mq_args(**over):
    a = dict(out=FAKE, ws=None, ws_bytes=0, q=FAKE, qs=FAKE, T=12, maxq=6, kc=FAKE, vc=FAKE,
             bt=FAKE, maxb=8, cl=FAKE, maxL=128, B=2, Hq=8, Hkv=2, D=64, bs=16, NB=64,
             scale=0.125, softcap=0.0, window=0, P=0, dt=_lib.PA_BF16, stream=None)
    a.update(over)
    return a


def call_mq(a):
    return _lib.load().pa_mq_attention(
        a["out"], a["ws"], a["ws_bytes"], a["q"], a["qs"], a["T"], a["maxq"], a["kc"], a["vc"],
        a["bt"], a["maxb"], a["cl"], a["maxL"], a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"],
        a["NB"], a["scale"], a["softcap"], a["window"], a["P"], a["dt"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(out=None), -1),
    (dict(qs=None), -1),
    (dict(cl=None), -1),
    (dict(B=0), -1),                      # tokens but no sequences
    (dict(maxq=0), -1),
    (dict(maxq=13), -1),                  # more than num_tokens
    (dict(T=-1), -1),
    (dict(Hq=6, Hkv=4), -1),
    (dict(maxL=129), -1),
    (dict(P=24), -1),
    (dict(softcap=-2.0), -1),
    (dict(D=80), -2),
    (dict(bs=24), -2),
    (dict(dt=_lib.PA_F32, Hq=6, Hkv=2), -2),   # per-token path: group of 3 not built
    (dict(), -3),                         # no workspace
    (dict(ws=FAKE, ws_bytes=64), -3),
])
def test_mq_rejects_bad_arguments(over, status):
    assert call_mq(mq_args(**over)) == status


def mq_step_args(rows=3, **over):
    a = mq_args(**over)
    s = _lib.MQStepArgs()
    s.key, s.value, s.slot_mapping, s.num_new_rows = FAKE, FAKE, FAKE, rows
    s.out, s.workspace, s.workspace_bytes, s.q = a["out"], a["ws"], a["ws_bytes"], a["q"]
    s.query_start, s.num_tokens, s.max_query_len = a["qs"], a["T"], a["maxq"]
    s.k_cache, s.v_cache, s.block_tables, s.max_blocks_per_seq = a["kc"], a["vc"], a["bt"], a["maxb"]
    s.context_lens, s.max_context_len, s.num_seqs = a["cl"], a["maxL"], a["B"]
    s.num_heads, s.num_kv_heads, s.head_dim, s.block_size = a["Hq"], a["Hkv"], a["D"], a["bs"]
    s.num_blocks, s.scale, s.softcap, s.window = a["NB"], a["scale"], a["softcap"], a["window"]
    s.partition_size, s.dtype = a["P"], a["dt"]
    return s


@pytest.mark.parametrize("rows,over,fields,status", [
    (-1, {}, {}, -1),
    (3, {}, dict(key=None), -1),
    (3, {}, dict(slot_mapping=None), -1),
    (3, dict(NB=0), {}, -1),
    (3, dict(bs=24), {}, -2),
    (3, dict(D=80), {}, -2),
    (3, dict(out=None), {}, -1),          # attention errors, checked before the fused launch
    (3, dict(maxq=13), {}, -1),
    (3, {}, {}, -3),                      # no workspace
    (0, {}, {}, -3),                      # no rows: pa_mq_attention alone
])
def test_mq_step_rejects_bad_arguments(rows, over, fields, status):
    """pa_mq_step reports the errors of pa_reshape_and_cache and
    pa_mq_attention before anything is enqueued."""
    a = mq_step_args(rows, **over)
    for k, v in fields.items():
        setattr(a, k, v)
    assert _lib.load().pa_mq_step(ctypes.byref(a), None) == status
    assert _lib.load().pa_mq_step(None, None) == -1


def test_mq_with_no_tokens_is_a_noop():
    assert call_mq(mq_args(T=0, maxq=0, out=None, q=None)) == 0


def test_mq_workspace_covers_the_decode_workspace_of_every_token():
    for B, T, L, P in ((4, 40, 300, 64), (512, 2560, 1024, 0), (1, 4096, 4096, 512)):
        assert (pa.mq_workspace_size(B, T, 8, 2, 128, L, P)
                >= pa.workspace_size(T, 8, 128, L, P) + 2 * T * 4)
    assert pa.mq_workspace_size(3, 0, 8, 2, 128, 300, 64) == 0


def test_mq_partition_choice_is_a_multiple_of_block_size():
    for bs in (1, 16, 32):
        for B, T, q, L in ((512, 2560, 5, 1024), (64, 575, 512, 4096), (4, 8192, 2048, 2048)):
            P = pa.mq_partition_size(B, T, q, 8, 4, 256, bs, L)
            assert P >= 0 and P % bs == 0


def test_static_step_refuses_oversize_before_any_gpu_call():
    """pa_step_static compares the step's scratch need with its static array
    before touching the GPU: an oversize request returns PA_ESCRATCH (-5)
    here, with no device present."""
    lib = _lib.load()
    a = _lib.StepArgs()
    a.out = a.q = a.k_cache = a.v_cache = a.block_tables = a.context_lens = FAKE
    a.num_seqs, a.num_heads, a.num_kv_heads, a.head_dim = 33, 32, 4, 256
    a.block_size, a.num_blocks, a.max_blocks_per_seq = 16, 100, 8192
    a.max_context_len, a.partition_size = 131072, 16
    a.scale, a.dtype = 0.125, _lib.PA_BF16
    assert pa.workspace_size(33, 32, 256, 131072, 16) > _lib.PA_STATIC_SCRATCH_BYTES
    assert lib.pa_step_static(ctypes.byref(a), None) == -5
    assert lib.pa_step_static(None, None) == -1
    assert pa.status_string(-5) not in ("ok", "unknown status")


def test_graph_of_steps_refuses_bad_arguments():
    """pa_step_graph_create_n checks its arguments before any capture: no
    steps, a null array or a null stream is PA_EINVAL (-1)."""
    lib = _lib.load()
    a = (_lib.StepArgs * 1)()
    h = ctypes.c_void_p()
    assert lib.pa_step_graph_create_n(a, 0, FAKE, ctypes.byref(h)) == -1
    assert lib.pa_step_graph_create_n(None, 1, FAKE, ctypes.byref(h)) == -1
    assert lib.pa_step_graph_create_n(a, 1, None, ctypes.byref(h)) == -1
    assert h.value is None


def test_decode_events_hook_arguments():
    """pa_set_decode_events takes both events or neither (no GPU call)."""
    lib = _lib.load()
    assert lib.pa_set_decode_events(FAKE, None) == -1
    assert lib.pa_set_decode_events(None, FAKE) == -1
    assert lib.pa_set_decode_events(None, None) == 0


def test_read_bandwidth_probe_refuses_bad_arguments():
    """pa_read_bandwidth_probe checks its arguments before any launch."""
    lib = _lib.load()
    assert lib.pa_read_bandwidth_probe(None, 1 << 20, 64, FAKE, None) == -1
    assert lib.pa_read_bandwidth_probe(FAKE, 1 << 20, 64, None, None) == -1
    assert lib.pa_read_bandwidth_probe(FAKE, 1 << 20, 0, FAKE, None) == -1
    assert lib.pa_read_bandwidth_probe(FAKE, 24, 64, FAKE, None) == -1     # not whole 16 B
    assert lib.pa_read_bandwidth_probe(FAKE, 0, 64, FAKE, None) == -1
    assert lib.pa_read_bandwidth_probe(FAKE + 8, 1 << 20, 64, FAKE, None) == -1  # misaligned
