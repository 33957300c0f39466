"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_kda_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = kda.lib()
    names = declared_functions()
    assert set(names) == set(kda.EXPORTS)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_version_and_sizes():
    assert kda.abi_version() == 5
    assert kda.state_bytes(96) == 96 * 128 * 128 * 4
    # the pages' per-request figure: 69 KDA layers x 12 heads per GPU at TP=8 x 128^2 x fp32
    assert abs(69 * kda.state_bytes(12) / 1e6 - 54.26) < 0.01
    assert kda.lib().kda_state_bytes(0) == 0


def test_status_strings():
    L = kda.lib()
    for s in range(5):
        assert L.kda_status_string(s)
    assert L.kda_status_string(99) == b"unknown status"


def test_config_defaults():
    c = kda.config(96)
    assert (c.num_heads, c.head_dim, c.io_dtype, c.out_dtype, c.prologue, c.epilogue, c.algo) == \
        (96, 128, kda.BF16, kda.BF16, 1, 1, 0)
    assert abs(c.scale - 128 ** -0.5) < 1e-7 and abs(c.l2_eps - 1e-6) < 1e-12
    assert (c.gate, c.gate_rank, c.beta_mode) == (0, 128, 0)


def test_config_struct_matches_header():
    """The Python mirror of kda_config has the header's fields in the header's order."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} kda_config;", text).group(1)
    names = re.findall(r"\b(\w+);", body)
    assert names == [f for f, _ in kda.Config._fields_]
    assert ctypes.sizeof(kda.Config) == 4 * len(names)


def test_beta_mode_validation():
    """beta_mode LOGIT passes validation (the call below stops at the missing workspace,
    before any launch); other values are refused."""
    c = kda.config(4, beta_mode="logit")
    assert c.beta_mode == 1
    assert _prefill(c, _args(workspace=None)) == kda.ERR_WORKSPACE_TOO_SMALL
    bad = kda.config(4)
    bad.beta_mode = 2
    assert _prefill(bad, _args(workspace=None)) == kda.ERR_INVALID_ARGUMENT
    assert kda.lib().kda_prefill_resolved_algo(ctypes.byref(bad), 1, 0) == -1


def test_workspace_size():
    c = kda.config(96)
    assert kda.workspace_size(c, 1, 100) == 0
    assert kda.workspace_size(c, 64, 10 ** 6) == 256
    assert kda.workspace_size(c, 65, 10) == 512
    with pytest.raises(kda.KdaError):
        kda.workspace_size(c, 0, 10)


FAKE = 0x10000  # aligned, never dereferenced: validation fails before any use


def _args(**over):
    a = kda.PrefillArgs()
    a.num_seqs, a.cu_seqlens, a.total_tokens = 2, FAKE, 10
    for f in ("q", "k", "v", "log_alpha", "beta", "g", "conv_w", "o", "state_out"):
        setattr(a, f, FAKE)
    a.workspace, a.workspace_bytes = FAKE, 256
    for k_, v_ in over.items():
        setattr(a, k_, v_)
    return a


def _prefill(cfg, a):
    return kda.lib().kda_prefill(ctypes.byref(cfg), ctypes.byref(a), None)


@pytest.mark.parametrize("field", ["cu_seqlens", "q", "k", "v", "log_alpha", "beta", "g", "o", "conv_w"])
def test_prefill_rejects_null_required(field):
    # a valid pointer everywhere except one required field, and a deliberately
    # too-small workspace as a second fault the check must not reach first
    assert _prefill(kda.config(4), _args(**{field: None})) == kda.ERR_INVALID_ARGUMENT


def test_prefill_rejects_misaligned():
    assert _prefill(kda.config(4), _args(q=FAKE + 2)) == kda.ERR_INVALID_ARGUMENT
    assert _prefill(kda.config(4), _args(state_in=FAKE + 8)) == kda.ERR_INVALID_ARGUMENT
    assert _prefill(kda.config(4), _args(state_in_slots=FAKE + 4)) == kda.ERR_INVALID_ARGUMENT
    assert _prefill(kda.config(4), _args(state_out_slots=FAKE + 4)) == kda.ERR_INVALID_ARGUMENT


def _header_fields(struct_name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^{}]*)\}\s*" + struct_name + ";", text).group(1)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if decl:
            names += [re.sub(r"[^A-Za-z0-9_]", "", part.split()[-1]) for part in decl.split(",")]
    return names


@pytest.mark.parametrize("cname, ctype", [("kda_config", kda.Config), ("kda_prefill_args", kda.PrefillArgs),
                                          ("kda_decode_args", kda.DecodeArgs)])
def test_binding_structs_match_header(cname, ctype):
    """The ctypes structures declare the header's fields in the header's order."""
    assert [f for f, _ in ctype._fields_] == _header_fields(cname)


def test_prefill_rejects_bad_config():
    assert kda.lib().kda_prefill(None, ctypes.byref(_args()), None) == kda.ERR_INVALID_ARGUMENT
    c = kda.config(4, head_dim=64)
    assert _prefill(c, _args()) == kda.ERR_UNSUPPORTED
    for field, val in (("num_heads", 0), ("io_dtype", 7), ("out_dtype", -1), ("prologue", 2),
                       ("algo", 9)):
        c = kda.config(4)
        setattr(c, field, val)
        assert _prefill(c, _args()) == kda.ERR_INVALID_ARGUMENT, field
    c = kda.config(4)
    c.rms_eps = -1.0
    assert _prefill(c, _args()) == kda.ERR_INVALID_ARGUMENT


def test_prefill_rejects_bad_sizes_and_workspace():
    assert _prefill(kda.config(4), _args(num_seqs=0)) == kda.ERR_INVALID_ARGUMENT
    assert _prefill(kda.config(4), _args(total_tokens=-1)) == kda.ERR_INVALID_ARGUMENT
    assert _prefill(kda.config(4), _args(workspace=None)) == kda.ERR_WORKSPACE_TOO_SMALL
    assert _prefill(kda.config(4), _args(workspace_bytes=8)) == kda.ERR_WORKSPACE_TOO_SMALL


def test_optional_pointers_follow_config():
    # g and conv_w are only required when the epilogue / prologue are on: with both
    # off a null g / conv_w passes those checks and the call fails on the workspace
    c = kda.config(4, prologue=False, epilogue=False)
    assert _prefill(c, _args(g=None, conv_w=None, workspace=None)) == kda.ERR_WORKSPACE_TOO_SMALL


def test_lowrank_gate_arguments():
    """With the low-rank gate log_alpha is optional and the four gate factors are
    required; bad ranks and the variants without the in-kernel gate are refused."""
    low = dict(gate_z=FAKE, gate_w=FAKE, gate_bias=FAKE, gate_a=FAKE)
    ok = kda.ERR_WORKSPACE_TOO_SMALL  # the next check after the pointer checks
    c = kda.config(4, gate="lowrank")
    assert _prefill(c, _args(log_alpha=None, workspace=None, **low)) == ok
    for f in low:
        assert _prefill(c, _args(log_alpha=None, **dict(low, **{f: None}))) == kda.ERR_INVALID_ARGUMENT, f
    # the log-alpha gate still requires log_alpha
    assert _prefill(kda.config(4), _args(log_alpha=None, **low)) == kda.ERR_INVALID_ARGUMENT
    for r in (0, 16, 48, 160):
        assert _prefill(kda.config(4, gate="lowrank", gate_rank=r), _args(**low)) == kda.ERR_UNSUPPORTED, r
    bad = kda.config(4)
    bad.gate = 5
    assert _prefill(bad, _args()) == kda.ERR_INVALID_ARGUMENT
    one = dict(num_seqs=1, workspace=None, workspace_bytes=0)
    assert _prefill(kda.config(4, gate="lowrank", algo="chunked_latency"), _args(**one, **low)) == kda.ERR_UNSUPPORTED
    assert _prefill(kda.config(4, gate="lowrank", io_dtype="f32", algo="chunked"),
                    _args(**one, **low)) == kda.ERR_UNSUPPORTED


@pytest.mark.parametrize("algo", ["chunked", "chunked_throughput", "chunked_scan", "chunked_latency"])
@pytest.mark.parametrize("gate", ["log_alpha", "head", "log_alpha_unbounded"])
def test_chunked_refuses_fp32_io(algo, gate):
    """The chunked kernels' split-bf16 products meet the bf16-input bar, not the fp32 one:
    they refuse fp32 io (and the retired latency variant refuses everything), while AUTO
    sends fp32 io to the recurrent kernel."""
    one = dict(num_seqs=1, workspace=FAKE, workspace_bytes=1 << 40)
    c = kda.config(4, io_dtype="f32", algo=algo, gate=gate)
    assert _prefill(c, _args(**one)) == kda.ERR_UNSUPPORTED
    assert kda.lib().kda_prefill_resolved_algo(ctypes.byref(c), 1, 64) == -1
    assert kda.resolved_algo(kda.config(4, io_dtype="f32", gate=gate), 1, 64) == "recurrent"


def test_decode_rejects_bad_arguments():
    L = kda.lib()

    def dec(cfg, **over):
        a = kda.DecodeArgs()
        a.batch = 4
        for f in ("q", "k", "v", "log_alpha", "beta", "g", "conv_w", "conv_state", "state", "o"):
            setattr(a, f, FAKE)
        for k_, v_ in over.items():
            setattr(a, k_, v_)
        return L.kda_decode_step(ctypes.byref(cfg), ctypes.byref(a), None)

    for f in ("q", "k", "v", "log_alpha", "beta", "g", "conv_w", "conv_state", "state", "o"):
        assert dec(kda.config(4), **{f: None}) == kda.ERR_INVALID_ARGUMENT, f
    assert dec(kda.config(4), batch=0) == kda.ERR_INVALID_ARGUMENT
    assert dec(kda.config(4), slots=FAKE + 4) == kda.ERR_INVALID_ARGUMENT
    assert dec(kda.config(4), slots_out=FAKE + 4) == kda.ERR_INVALID_ARGUMENT
    assert dec(kda.config(4, head_dim=256)) == kda.ERR_UNSUPPORTED


def test_scan_grid_limit():
    """A named segmented prefill whose grids would not fit one 32-bit dimension (8 x N x H
    workgroups for the scan) is refused after the workspace check and before any HIP call."""
    n = 3_000_000  # 3M one-token sequences x 96 heads: 288M items, 2.3G scan workgroups
    a = _args(num_seqs=n, total_tokens=n, workspace_bytes=1 << 62)
    assert _prefill(kda.config(96, algo="chunked_scan"), a) == kda.ERR_UNSUPPORTED


def test_no_alloc_validation():
    """kda_prefill_no_alloc validates like kda_prefill and ignores the caller's workspace;
    a configuration whose workspace exceeds the static scratch (the segmented prefill, when
    named: AUTO never selects it here) is refused before any HIP call.  Only refusals are
    exercised: these arguments hold no device memory."""
    L = kda.lib()

    def na(cfg, a):
        return L.kda_prefill_no_alloc(ctypes.byref(cfg), ctypes.byref(a), None)

    assert na(kda.config(4, algo="chunked_scan"), _args(num_seqs=3, total_tokens=300)) == kda.ERR_WORKSPACE_TOO_SMALL
    assert na(kda.config(4), _args(q=None)) == kda.ERR_INVALID_ARGUMENT
    assert na(kda.config(4), _args(num_seqs=0)) == kda.ERR_INVALID_ARGUMENT
    assert na(kda.config(4, head_dim=64), _args()) == kda.ERR_UNSUPPORTED
    assert na(kda.config(4, io_dtype="f32", algo="chunked_throughput"), _args(num_seqs=1)) == kda.ERR_UNSUPPORTED


def test_resolved_algo():
    # fp32 io -> the recurrent reference path; explicit choices pass through;
    # invalid configurations and sequence counts -> -1
    L = kda.lib()
    c = kda.config(4, io_dtype="f32")
    assert kda.resolved_algo(c, 3) == "recurrent"
    for name in ("recurrent", "chunked_throughput"):
        assert kda.resolved_algo(kda.config(4, algo=name), 2) == name
    assert L.kda_prefill_resolved_algo(ctypes.byref(kda.config(4, algo="chunked_latency")), 2, 0) == -1
    assert kda.resolved_algo(kda.config(8), 1) == "chunked_throughput"
    assert kda.resolved_algo(kda.config(96, algo="chunked"), 4) == "chunked_throughput"
    assert L.kda_prefill_resolved_algo(ctypes.byref(kda.config(4)), 0, 0) == -1
    assert L.kda_prefill_resolved_algo(ctypes.byref(kda.config(4)), 1, -1) == -1
    bad = kda.config(4)
    bad.algo = 9
    assert L.kda_prefill_resolved_algo(ctypes.byref(bad), 1, 0) == -1


def test_scan_selection_and_workspace():
    """AUTO splits the sequences when one pass would leave most compute units idle (256
    when sized without a device): at most 96 (sequence, head) items over sequences
    averaging 1024 tokens or more, or at most 128 items over sequences averaging 16384;
    the workspace then holds two 64 KiB matrices per (segment slot, head)."""
    c = kda.config(96)
    assert kda.resolved_algo(c, 1, 131072) == "chunked_scan"
    assert kda.resolved_algo(c, 4, 16384) == "chunked_throughput"     # 384 items
    assert kda.resolved_algo(c, 1, 8192) == "chunked_scan"            # 96 items
    assert kda.resolved_algo(c, 1, 1023) == "chunked_throughput"      # too short
    assert kda.resolved_algo(kda.config(12), 4, 4 * 4096) == "chunked_scan"   # 48 items
    assert kda.resolved_algo(kda.config(128), 1, 8192) == "chunked_throughput"  # 128 items
    assert kda.resolved_algo(kda.config(128), 1, 16384) == "chunked_scan"       # long
    assert kda.resolved_algo(kda.config(192), 1, 32768) == "chunked_throughput"  # 192 items
    assert kda.resolved_algo(kda.config(96), 2, 2 * 16384) == "chunked_throughput"
    assert kda.resolved_algo(kda.config(96, gate="head"), 1, 8192) == "chunked_scan"
    assert kda.resolved_algo(kda.config(96, io_dtype="f32"), 1, 131072) == "recurrent"
    assert kda.resolved_algo(kda.config(96, gate="lowrank_softplus"), 1, 131072) == "chunked_throughput"
    assert kda.resolved_algo(kda.config(96, algo="chunked_throughput"), 1, 131072) == "chunked_throughput"
    # one 131072-token sequence x 96 heads: 6 segments of 21856 tokens (5 reruns x 96 heads
    # fill two workgroup slots on each of 256 CUs), 7 slots
    assert kda.workspace_size(c, 1, 131072) == 256 + 256 + 2 * 7 * 96 * 128 * 128 * 4
    # P segments with P - 1 = floor(512 / items): the rerun pass fills two workgroup slots on
    # each of 256 CUs (12 heads: 43 segments of 3056 tokens, 44 slots; 48 heads: 11 of 11920)
    for heads, segs in ((12, 43), (48, 11), (32, 17)):
        seg = -(-(-(-131072 // segs)) // 16) * 16
        assert (131072 + seg - 1) // seg == segs
        table = -(-(1 + segs) * 32 // 256) * 256  # one 32-byte descriptor per slot, 256-byte aligned
        assert kda.workspace_size(kda.config(heads), 1, 131072) == table + 256 + 2 * (1 + segs) * heads * 128 * 128 * 4
    # named: segments of at least 64 tokens (3 x 100 tokens, 2 heads: 3 + 5 slots)
    s = kda.config(2, algo="chunked_scan")
    assert kda.workspace_size(s, 3, 300) == 256 + 256 + 2 * 8 * 2 * 128 * 128 * 4
    one = dict(num_seqs=1, workspace=None, workspace_bytes=0)
    big = dict(num_seqs=1, workspace=FAKE, workspace_bytes=1 << 40)
    assert _prefill(kda.config(4, algo="chunked_scan", io_dtype="f32"), _args(**big)) == kda.ERR_UNSUPPORTED
    assert _prefill(kda.config(4, algo="chunked_scan", gate="log_alpha_unbounded"), _args(**big)) == kda.ERR_UNSUPPORTED


def test_head_gate_arguments():
    """The scalar per-head gate reads log_alpha [T, H]: it is required, the low-rank
    factors are ignored, and only the recurrent and throughput kernels take it."""
    c = kda.config(4, gate="head")
    assert c.gate == 2
    assert _prefill(c, _args(log_alpha=None)) == kda.ERR_INVALID_ARGUMENT
    assert _prefill(c, _args(workspace=None)) == kda.ERR_WORKSPACE_TOO_SMALL
    one = dict(num_seqs=1, workspace=None, workspace_bytes=0)
    assert _prefill(kda.config(4, gate="head", algo="chunked_latency"), _args(**one)) == kda.ERR_UNSUPPORTED
    assert kda.resolved_algo(kda.config(4, gate="head"), 1) == "chunked_throughput"


def test_unbounded_gate_arguments():
    """Kimi Linear's softplus gate takes the low-rank factors like the K3 gate; log alpha
    without a floor is required like log alpha; neither runs on the pipelined variant."""
    low = dict(gate_z=FAKE, gate_w=FAKE, gate_bias=FAKE, gate_a=FAKE)
    c = kda.config(4, gate="lowrank_softplus")
    assert c.gate == 3
    assert _prefill(c, _args(log_alpha=None, workspace=None, **low)) == kda.ERR_WORKSPACE_TOO_SMALL
    assert _prefill(c, _args(log_alpha=None, gate_w=None, **{k: v for k, v in low.items() if k != "gate_w"})) \
        == kda.ERR_INVALID_ARGUMENT
    assert _prefill(kda.config(4, gate="lowrank_softplus", gate_rank=48), _args(**low)) == kda.ERR_UNSUPPORTED
    u = kda.config(4, gate="log_alpha_unbounded")
    assert u.gate == 4
    assert _prefill(u, _args(log_alpha=None)) == kda.ERR_INVALID_ARGUMENT
    assert _prefill(u, _args(workspace=None)) == kda.ERR_WORKSPACE_TOO_SMALL
    one = dict(num_seqs=1, workspace=None, workspace_bytes=0)
    for g in ("lowrank_softplus", "log_alpha_unbounded"):
        assert _prefill(kda.config(4, gate=g, algo="chunked_latency"), _args(**one, **low)) == kda.ERR_UNSUPPORTED, g
    bad = kda.config(4)
    bad.gate = 5
    assert _prefill(bad, _args()) == kda.ERR_INVALID_ARGUMENT


def test_binding_refuses_tensors_off_the_gpu():
    """The binding passes raw pointers: a host tensor is refused before any library call."""
    import torch
    T, H = 16, 2
    bf = torch.bfloat16
    q, k, v, g = (torch.zeros((T, H, 128), dtype=bf) for _ in range(4))
    la = torch.zeros((T, H, 128), dtype=torch.float32)
    beta = torch.zeros((T, H), dtype=torch.float32)
    cu = torch.tensor([0, T], dtype=torch.int32)
    cw = torch.zeros((3, H * 128, 4), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensors"):
        kda.prefill(q, k, v, la, beta, cu, g=g, conv_w=cw)
    st = torch.zeros((T, H, 128, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensors"):
        kda.decode_step(q, k, v, la, beta, st, g=g, conv_w=cw, conv_state=torch.zeros((T, 3, 3, H * 128), dtype=bf))
