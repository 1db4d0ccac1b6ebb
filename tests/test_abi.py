"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/*.h declares, and rejects invalid arguments on the host before
any HIP call (nothing is enqueued, so no device is needed)."""
import ctypes
import glob
import os
import re

import pytest

from mxfp4_routed_expert_sqrt_amd import capi
from mxfp4_routed_expert_sqrt_amd.configs import SHAPES, MoEShape
from mxfp4_routed_expert_sqrt_amd.layer import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = capi.lib()
    names = declared_functions()
    assert "moe_layer_forward" in names and "moe_workspace_size" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(capi.EXPORTED)


def test_hbm_probe_library_exports_its_header_and_checks_arguments():
    # include/hbm_probe.h belongs to the streaming-read probe (libmoe_hbm.so), not to the layer's library
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "hbm_probe.h")).read(), flags=re.S)
    names = set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(hbm_\w+)\s*\(", text, flags=re.M))
    assert names == {"hbm_read_probe", "hbm_probe_sink_words"}
    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_routed_expert_sqrt_amd", "libmoe_hbm.so"))
    for n in names:
        assert hasattr(lib, n), n
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.hbm_probe_sink_words.argtypes = [ctypes.c_int]
    assert lib.hbm_probe_sink_words(10) == 40
    # rejected on the host before any launch: no buffer, a size that is not whole 16-byte pieces,
    # a misaligned start, no workgroups
    fake = 1 << 20
    assert lib.hbm_read_probe(None, 1024, 0, fake, 4, None) == -1
    assert lib.hbm_read_probe(fake, 1000, 0, fake, 4, None) == -1
    assert lib.hbm_read_probe(fake + 8, 1024, 0, fake, 4, None) == -1
    assert lib.hbm_read_probe(fake, 1024, 0, fake, 0, None) == -1


def test_version_and_status_strings():
    assert capi.moe_version() == 5
    for st in (0, -1, -2, -3, -4, -5):
        assert capi.moe_status_string(st) != "unknown status"
    assert capi.moe_status_string(7) == "unknown status"


def test_packed_sizes():
    # q keeps the natural byte count; scales are padded to whole 4-k-step groups
    assert capi.moe_packed_mxfp4_bytes(2048, 4096) == (2048 * 2048, 128 * 8 * 256)
    assert capi.moe_packed_mxfp4_bytes(4096, 2048) == (4096 * 1024, 256 * 4 * 256)
    assert capi.moe_packed_mxfp4_bytes(128, 256) == (128 * 128, 8 * 1 * 256)
    with pytest.raises(capi.MoeError):
        capi.moe_packed_mxfp4_bytes(24, 256)
    with pytest.raises(capi.MoeError):
        capi.moe_packed_mxfp4_bytes(32, 96)


def test_workspace_size_arithmetic():
    sh = SHAPES["verify512"]
    cfg = make_config(sh)
    b = capi.moe_workspace_size(cfg, 512)
    N, k, E, d, I = 512, 6, 256, 4096, 2048
    Ptot = N * k + N
    # the big regions: fp32 y, split h, split x, the normalised input, router logits (1 to 16 split-K partials)
    assert b >= Ptot * d * 4 + Ptot * I * 2 + N * d * 2 + N * d * 2 + N * E * 4
    assert b < (Ptot * d * 4 + Ptot * I * 2 + N * d * 2 + N * d * 2 + 16 * N * E * 4) * 1.05
    assert capi.moe_workspace_size(cfg, 0) == 0
    assert capi.moe_workspace_size(cfg, 1024) > b


@pytest.mark.parametrize("field,value,status", [
    ("d_model", 96, capi.MOE_ERR_UNSUPPORTED), ("d_ff", 200, capi.MOE_ERR_UNSUPPORTED),
    ("n_experts", 0, capi.MOE_ERR_UNSUPPORTED), ("n_experts", 1025, capi.MOE_ERR_UNSUPPORTED),
    ("top_k", 0, capi.MOE_ERR_UNSUPPORTED), ("top_k", 9, capi.MOE_ERR_UNSUPPORTED),
    ("routing", 2, capi.MOE_ERR_INVALID), ("has_shared", 3, capi.MOE_ERR_INVALID),
    ("norm_eps", -1e-6, capi.MOE_ERR_INVALID), ("norm_eps", float("inf"), capi.MOE_ERR_INVALID),
    ("norm_eps", float("nan"), capi.MOE_ERR_INVALID), ("bias_mode", 2, capi.MOE_ERR_INVALID),
    ("bias_mode", -1, capi.MOE_ERR_INVALID), ("shared_format", 2, capi.MOE_ERR_INVALID),
    ("shared_format", -1, capi.MOE_ERR_INVALID), ("expert_format", 2, capi.MOE_ERR_INVALID),
    ("expert_format", -1, capi.MOE_ERR_INVALID),
    # Q2_K experts with the MXFP4 shared expert, or widths that are not whole super-blocks
    ("expert_format", capi.MOE_EXPERTS_Q2K, capi.MOE_ERR_UNSUPPORTED),
])
def test_bad_config_rejected(field, value, status):
    cfg = make_config(SHAPES["tiny"])
    setattr(cfg, field, value)
    b = ctypes.c_size_t()
    assert capi.lib().moe_workspace_size(ctypes.byref(cfg), 32, ctypes.byref(b)) == status
    args = capi.MoeArgs()
    args.n_rows = 32
    assert capi.moe_layer_forward(cfg, args, None) == status


def _valid_args(cfg, N):
    """Arguments with plausible (never dereferenced) aligned addresses."""
    a = capi.MoeArgs()
    a.n_rows = N
    a.x, a.router_w, a.out = 0x10000000, 0x20000000, 0x30000000
    w = capi.MoeWeights()
    for i, name in enumerate(n for n, _ in capi.MoeWeights._fields_):
        setattr(w, name, 0x40000000 + i * 0x1000000)
    a.w = w
    a.workspace = 0x80000000
    a.workspace_bytes = capi.moe_workspace_size(cfg, N) if N else 0
    return a


def test_invalid_arguments_return_before_any_hip_call():
    cfg = make_config(SHAPES["tiny"])
    N = 32
    cases = []
    a = _valid_args(cfg, N); a.x = None; cases.append((a, capi.MOE_ERR_INVALID))
    a = _valid_args(cfg, N); a.out = 0x30000008; cases.append((a, capi.MOE_ERR_INVALID))     # misaligned
    a = _valid_args(cfg, N); a.out = a.x + 64; cases.append((a, capi.MOE_ERR_INVALID))       # overlaps x
    a = _valid_args(cfg, N); a.w.down_s = None; cases.append((a, capi.MOE_ERR_INVALID))
    a = _valid_args(cfg, N); a.w.sh_up_q = 0x50000004; cases.append((a, capi.MOE_ERR_INVALID))
    a = _valid_args(cfg, N); a.workspace_bytes -= 1; cases.append((a, capi.MOE_ERR_WORKSPACE))
    a = _valid_args(cfg, N); a.workspace = None; cases.append((a, capi.MOE_ERR_WORKSPACE))
    a = _valid_args(cfg, N); a.workspace = 0x80000080; cases.append((a, capi.MOE_ERR_INVALID))
    a = _valid_args(cfg, N); a.perm = 0x90000002; cases.append((a, capi.MOE_ERR_INVALID))
    a = _valid_args(cfg, N); a.n_rows = -1; cases.append((a, capi.MOE_ERR_INVALID))
    a = _valid_args(cfg, N); a.n_rows = capi.MOE_MAX_ROWS + 1; cases.append((a, capi.MOE_ERR_UNSUPPORTED))
    a = _valid_args(cfg, N); a.norm_w = 0xA0000008; cases.append((a, capi.MOE_ERR_INVALID))   # misaligned
    a = _valid_args(cfg, N); a.residual = 0xB0000004; cases.append((a, capi.MOE_ERR_INVALID))  # misaligned
    a = _valid_args(cfg, N); a.residual = a.out + 512; cases.append((a, capi.MOE_ERR_INVALID))  # partial overlap
    a = _valid_args(cfg, N); a.x = a.workspace + 256; cases.append((a, capi.MOE_ERR_INVALID))     # x in workspace
    a = _valid_args(cfg, N); a.router_w = a.workspace; cases.append((a, capi.MOE_ERR_INVALID))
    a = _valid_args(cfg, N); a.residual = a.workspace + 4096; cases.append((a, capi.MOE_ERR_INVALID))
    for a, st in cases:
        assert capi.moe_layer_forward(cfg, a, None) == st
    hcfg = make_config(SHAPES["hash2048"])
    a = _valid_args(hcfg, 8)
    assert capi.moe_layer_forward(hcfg, a, None) == capi.MOE_ERR_INVALID  # hash mode without a table
    bcfg = make_config(SHAPES["tiny"], shared_format=capi.MOE_SHARED_BF16)
    for field, value in (("sh_up_w", None), ("sh_down_w", 0x4C000008), ("sh_gate_w", None)):
        a = _valid_args(bcfg, N); setattr(a.w, field, value)
        assert capi.moe_layer_forward(bcfg, a, None) == capi.MOE_ERR_INVALID, field
    a = _valid_args(bcfg, N); a.w.sh_gate_w = a.workspace + 512
    assert capi.moe_layer_forward(bcfg, a, None) == capi.MOE_ERR_INVALID  # bf16 shared weights in the workspace
    a = _valid_args(bcfg, N); a.w.sh_gate_q = None; a.w.sh_down_s = None
    a.workspace_bytes = 0
    assert capi.moe_layer_forward(bcfg, a, None) == capi.MOE_ERR_WORKSPACE  # MXFP4 shared pointers not needed
    nosh = make_config(SHAPES["tiny"], has_shared=False)
    a = _valid_args(nosh, N); a.w.sh_gate_q = None
    a.workspace_bytes = 0
    assert capi.moe_layer_forward(nosh, a, None) == capi.MOE_ERR_WORKSPACE  # shared pointers not needed


def test_every_written_buffer_is_disjoint_from_the_others():
    # out, the workspace and the optional routing outputs are written; none may overlap any buffer of
    # the call (weights, hash tables, routing outputs included), or the call is rejected before any
    # HIP call.  Reads may overlap each other.
    cfg = make_config(SHAPES["tiny"])
    N, E, k = 32, 16, 2
    cases = []
    a = _valid_args(cfg, N); a.w.gate_q = a.workspace + 256; cases.append(("weights in workspace", a))
    a = _valid_args(cfg, N); a.w.down_s = a.out + 64; cases.append(("scales under out", a))
    a = _valid_args(cfg, N); a.w.sh_up_q = a.workspace + 4096; cases.append(("shared weights in workspace", a))
    a = _valid_args(cfg, N); a.topk_idx = a.out; cases.append(("topk_idx on out", a))
    a = _valid_args(cfg, N); a.perm = a.x + 16; cases.append(("perm on x", a))
    a = _valid_args(cfg, N); a.counts = 0x90000000; a.offsets = 0x90000000 + 4 * (E - 1)
    cases.append(("counts and offsets overlap", a))
    a = _valid_args(cfg, N); a.inv = a.workspace + 1024; cases.append(("inv in workspace", a))
    a = _valid_args(cfg, N); a.topk_w = a.w.up_s; cases.append(("gates on weight scales", a))
    for label, a in cases:
        assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_INVALID, label
    # hash mode: the token ids and the whole table are read
    hsh = MoEShape("edge_hash", 50, 256, 16, 2, 128, "hash", "tiny", vocab=97)
    hcfg = make_config(hsh)
    a = _valid_args(hcfg, 50); a.token_ids, a.tid2eid, a.vocab = 0xC0000000, 0xD0000000, 97
    a.workspace_bytes -= 1
    assert capi.moe_layer_forward(hcfg, a, None) == capi.MOE_ERR_WORKSPACE  # valid up to the workspace size
    a.workspace_bytes += 1
    a.tid2eid = a.workspace + a.workspace_bytes - 8  # the table's first row is inside, the rest beyond
    assert capi.moe_layer_forward(hcfg, a, None) == capi.MOE_ERR_INVALID
    a.tid2eid, a.token_ids = 0xD0000000, a.out + 50 * 256 * 2 - 4  # the ids' first entry is out's last 4 bytes
    assert capi.moe_layer_forward(hcfg, a, None) == capi.MOE_ERR_INVALID
    # reads overlapping each other are allowed: residual == x, gate and up scales shared
    a = _valid_args(cfg, N); a.residual = a.x; a.w.up_s = a.w.gate_s; a.workspace_bytes -= 1
    assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_WORKSPACE


Q2K_TINY = MoEShape("tiny_q2k", 32, 256, 16, 2, 256, "topk", "tiny_q2k")


def test_q2k_config_and_sizes():
    assert capi.moe_q2k_bytes(2048, 4096) == 2048 * 16 * 84
    assert capi.moe_q2k_bytes(16, 256) == 16 * 84
    for rows, K in ((24, 256), (16, 128), (16, 384 + 64)):
        with pytest.raises(capi.MoeError):
            capi.moe_q2k_bytes(rows, K)
    ok = make_config(Q2K_TINY, shared_format=capi.MOE_SHARED_BF16, expert_format=capi.MOE_EXPERTS_Q2K)
    assert capi.moe_workspace_size(ok, 32) > 0
    assert capi.moe_workspace_size(make_config(Q2K_TINY, has_shared=False, expert_format=capi.MOE_EXPERTS_Q2K), 32) > 0
    b = ctypes.c_size_t()
    for shape, shared, fmt in ((SHAPES["tiny"], True, capi.MOE_SHARED_BF16),  # I = 128
                               (Q2K_TINY, True, capi.MOE_SHARED_MXFP4),
                               (MoEShape("q2k_d384", 32, 384, 16, 2, 256, "topk", "x"), False, 0)):
        cfg = make_config(shape, has_shared=shared, shared_format=fmt, expert_format=capi.MOE_EXPERTS_Q2K)
        assert capi.lib().moe_workspace_size(ctypes.byref(cfg), 32, ctypes.byref(b)) == capi.MOE_ERR_UNSUPPORTED


def test_q2k_arguments_checked_before_any_hip_call():
    cfg = make_config(Q2K_TINY, shared_format=capi.MOE_SHARED_BF16, expert_format=capi.MOE_EXPERTS_Q2K)
    N = 32
    # the scale pointers are not used: absent scales are fine (valid up to the workspace size)
    a = _valid_args(cfg, N)
    for n in ("gate_s", "up_s", "down_s", "sh_gate_q", "sh_gate_s", "sh_up_q", "sh_up_s", "sh_down_q", "sh_down_s"):
        setattr(a.w, n, None)
    a.workspace_bytes -= 1
    assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_WORKSPACE
    for field, value in (("gate_q", None), ("up_q", 0x41000008), ("down_q", None)):
        a = _valid_args(cfg, N); setattr(a.w, field, value)
        assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_INVALID, field
    # a Q2_K weight set is E * rows * K/256 * 84 bytes: one byte short of the workspace is still an overlap
    a = _valid_args(cfg, N)
    a.w.down_q = a.workspace - 16 * 256 * 84 + 16
    assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_INVALID
    a.w.down_q = a.workspace - 16 * 256 * 84
    a.workspace_bytes -= 1
    assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_WORKSPACE
    # the packing entry point
    assert capi.moe_pack_q2k(None, 0, 16, 256, None, None) == capi.MOE_OK
    assert capi.moe_pack_q2k(0x1000, 1, 16, 256, None, None) == capi.MOE_ERR_INVALID
    assert capi.moe_pack_q2k(0x1002, 1, 16, 256, 0x9000, None) == capi.MOE_ERR_INVALID   # q not 4-aligned
    assert capi.moe_pack_q2k(0x1000, 1, 16, 256, 0x9008, None) == capi.MOE_ERR_INVALID   # out not 16-aligned
    assert capi.moe_pack_q2k(0x1000, 1, 16, 256, 0x1100, None) == capi.MOE_ERR_INVALID   # overlap
    assert capi.moe_pack_q2k(0x1000, 1, 16, 200, 0x9000, None) == capi.MOE_ERR_UNSUPPORTED
    assert capi.moe_pack_q2k(0x1000, -1, 16, 256, 0x9000, None) == capi.MOE_ERR_INVALID


def test_zero_rows_is_a_no_op():
    cfg = make_config(SHAPES["tiny"])
    a = capi.MoeArgs()
    a.n_rows = 0
    assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_OK


def test_pack_rejects_bad_arguments():
    L = capi.lib()
    assert capi.moe_pack_mxfp4(None, None, 0, 16, 128, None, None, None) == capi.MOE_OK
    assert capi.moe_pack_mxfp4(None, 0x1000, 1, 16, 128, 0x2000, 0x3000, None) == capi.MOE_ERR_INVALID
    assert capi.moe_pack_mxfp4(0x1000, 0x2000, 1, 20, 128, 0x3000, 0x4000, None) == capi.MOE_ERR_UNSUPPORTED
    assert capi.moe_pack_mxfp4(0x1008, 0x2000, 1, 16, 128, 0x3000, 0x4000, None) == capi.MOE_ERR_INVALID
    assert capi.moe_pack_mxfp4(0x1000, 0x2000, 1, 16, 128, 0x1200, 0x4000, None) == capi.MOE_ERR_INVALID  # overlap
    assert L is not None


def test_bf16_pack_and_packed_shared_expert_are_checked_before_any_hip_call():
    # moe_pack_bf16: sizes, alignment, overlap
    assert capi.moe_pack_bf16(None, 0, 16, 32, None, None) == capi.MOE_OK
    assert capi.moe_pack_bf16(None, 1, 16, 32, 0x2000, None) == capi.MOE_ERR_INVALID
    assert capi.moe_pack_bf16(0x1000, 1, 24, 32, 0x9000, None) == capi.MOE_ERR_UNSUPPORTED   # rows % 16
    assert capi.moe_pack_bf16(0x1000, 1, 16, 48, 0x9000, None) == capi.MOE_ERR_UNSUPPORTED   # K % 32
    assert capi.moe_pack_bf16(0x1008, 1, 16, 32, 0x9000, None) == capi.MOE_ERR_INVALID       # w not 16-aligned
    assert capi.moe_pack_bf16(0x1000, 1, 16, 32, 0x9008, None) == capi.MOE_ERR_INVALID       # out not 16-aligned
    assert capi.moe_pack_bf16(0x1000, 1, 16, 32, 0x1000 + 16 * 32 * 2 - 16, None) == capi.MOE_ERR_INVALID  # overlap
    assert capi.moe_pack_bf16(0x1000, -1, 16, 32, 0x9000, None) == capi.MOE_ERR_INVALID
    # moe_args_t.sh_packed with a bf16 shared expert: 16-byte aligned, read over 3*I*d*2 bytes
    cfg = make_config(SHAPES["tiny"], shared_format=capi.MOE_SHARED_BF16)
    N, d, I = 32, 256, 128
    a = _valid_args(cfg, N); a.sh_packed = 0xE0000008
    assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_INVALID
    a = _valid_args(cfg, N); a.sh_packed = a.workspace - 3 * I * d * 2 + 16   # its last 16 bytes in the workspace
    assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_INVALID
    a.sh_packed = a.workspace - 3 * I * d * 2
    a.workspace_bytes -= 1
    assert capi.moe_layer_forward(cfg, a, None) == capi.MOE_ERR_WORKSPACE     # valid up to the workspace size
    # with the MXFP4 shared expert the field is not read
    mcfg = make_config(SHAPES["tiny"])
    a = _valid_args(mcfg, N); a.sh_packed = 0xE0000008; a.workspace_bytes -= 1
    assert capi.moe_layer_forward(mcfg, a, None) == capi.MOE_ERR_WORKSPACE


def test_binding_structs_match_the_c_header(tmp_path):
    # offsets and sizes of every field of the three ABI structs, as the C compiler lays them out
    # from include/moe_mxfp4.h, against the ctypes mirrors; and the header's constants
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    structs = {"moe_config_t": capi.MoeConfig, "moe_weights_t": capi.MoeWeights, "moe_args_t": capi.MoeArgs}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "moe_mxfp4.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    consts = ["MOE_OK", "MOE_ERR_INVALID", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP",
              "MOE_ROUTING_TOPK", "MOE_ROUTING_HASH", "MOE_BIAS_LOGIT", "MOE_BIAS_SELECT", "MOE_SHARED_MXFP4",
              "MOE_SHARED_BF16", "MOE_MAX_ROWS", "MOE_ERR_SCRATCH", "MOE_NOALLOC_SCRATCH_BYTES",
              "MOE_N_STAGES", "MOE_N_STAGE_EVENTS", "MOE_MXFP4_VERSION", "MOE_EXPERTS_MXFP4", "MOE_EXPERTS_Q2K",
              "MOE_SHARED_STREAM_ROWS"]
    for c in consts:
        lines.append(f'  printf("const {c} %ld\\n", (long)({c}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c99", "-I", inc, "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    seen = 0
    for line in filter(None, out):
        kind, name, value = line.split()
        value = int(value)
        if kind == "const":
            want = getattr(capi, name) if name != "MOE_MXFP4_VERSION" else capi.moe_version()
            assert value == want, name
        elif name == "sizeof":
            assert value == ctypes.sizeof(structs[kind]), kind
        else:
            assert value == getattr(structs[kind], name).offset, f"{kind}.{name}"
        seen += 1
    assert seen == len(consts) + sum(len(c._fields_) + 1 for c in structs.values())
