"""GPU parity of the serving-state features against the fp64 oracle, through the C ABI:
slot-indexed state and conv-cache pools in prefill, copy-on-write forks from read-only
checkpoints in prefill and decode ("Kimi K3: Architecture and SGLang Day-0 Support",
section "RadixAttention: prefix caching for KDA state"), and speculative verification of
draft tokens followed by a replay of the accepted ones ("Inside Kimi K3: How KDA, AttnRes,
and 896 Experts Work", section "What could go wrong").

The oracle has no notion of pools: it runs on the rows a call reads (gathered on the host),
and the pool rows a call writes are compared with its results.  Rows a call does not write
must come back bit for bit.
"""
import numpy as np
import pytest

import kda_workloads as W
from kda_testlib import err, oracle_prefill, say, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = {"recurrent": 1e-4, "chunked_throughput": 1e-2, "auto": 1e-2}
H = 2
HD = H * W.D


def _pools(rows, seed):
    rng = np.random.default_rng(seed)
    st = (rng.standard_normal((rows, H, W.D, W.D)) * 0.02).astype(np.float32)
    cv = W.bf16_round(rng.standard_normal((rows, 3, 3, HD)).astype(np.float32))
    return st, cv


def _dev_prefill(inp, st_pool, cv_pool, algo, in_slots=None, out_slots=None, write=True):
    """kda_prefill on device pools (state and conv updated in place when `write`)."""
    import torch
    import gated_delta_rule_kda_amd as kda
    bf = torch.bfloat16
    cfg = kda.config(H, io_dtype="bf16", out_dtype="f32", prologue=True, epilogue=True, algo=algo)
    o, _, _ = kda.prefill(
        to_dev(inp["q"], bf), to_dev(inp["k"], bf), to_dev(inp["v"], bf),
        to_dev(inp["log_alpha"], torch.float32), to_dev(inp["beta"], torch.float32),
        to_dev(inp["cu_seqlens"].astype(np.int32), torch.int32), g=to_dev(inp["g"], bf),
        conv_w=to_dev(inp["conv_w"], torch.float32), conv_in=cv_pool, state_in=st_pool,
        conv_out=cv_pool if write else None, state_out=st_pool if write else None,
        state_in_slots=None if in_slots is None else to_dev(np.asarray(in_slots, np.int32), torch.int32),
        state_out_slots=None if out_slots is None else to_dev(np.asarray(out_slots, np.int32), torch.int32),
        cfg=cfg, return_state=False, return_conv=False)
    torch.cuda.synchronize()
    return to_np(o)


@pytest.mark.parametrize("algo", ["recurrent", "chunked_throughput"])
def test_prefill_reads_and_writes_pool_rows(algo):
    """Three sequences (one of them empty) read pool rows 5, 2, 0 and write rows 1, 6, 3 of
    the same state and conv pools; every other row is left untouched."""
    import torch
    inp = W.gen_prefill(W.PrefillSpec(lens=[37, 0, 70], heads=H, seed=61))
    rows, ins, outs = 8, [5, 2, 0], [1, 6, 3]
    st, cv = _pools(rows, 62)
    ref_in = dict(inp, state_in=st[ins], conv_in=cv[ins])
    r = oracle_prefill(ref_in)
    st_d, cv_d = to_dev(st, torch.float32), to_dev(cv, torch.bfloat16)
    say(f"pool prefill {algo}")
    o = _dev_prefill(inp, st_d, cv_d, algo, ins, outs)
    st_n, cv_n = to_np(st_d), to_np(cv_d)
    assert err(o, r["o"]) <= TOL[algo]
    assert err(st_n[outs], r["state"]) <= TOL[algo]
    assert np.array_equal(cv_n[outs], r["conv"])
    # the empty sequence copies its row through exactly
    assert np.array_equal(st_n[6], st[2].astype(np.float64))
    keep = [i for i in range(rows) if i not in outs]
    assert np.array_equal(st_n[keep], st[keep].astype(np.float64))
    assert np.array_equal(cv_n[keep], cv[keep].astype(np.float64))


def test_prefill_copy_on_write_fork():
    """Two sequences fork one read-only prefix checkpoint (row 3) into rows 0 and 5."""
    import torch
    inp = W.gen_prefill(W.PrefillSpec(lens=[20, 45], heads=H, seed=63))
    rows, ins, outs = 6, [3, 3], [0, 5]
    st, cv = _pools(rows, 64)
    r = oracle_prefill(dict(inp, state_in=st[ins], conv_in=cv[ins]))
    st_d, cv_d = to_dev(st, torch.float32), to_dev(cv, torch.bfloat16)
    o = _dev_prefill(inp, st_d, cv_d, "auto", ins, outs)
    st_n, cv_n = to_np(st_d), to_np(cv_d)
    assert err(o, r["o"]) <= TOL["auto"]
    assert err(st_n[outs], r["state"]) <= TOL["auto"]
    assert np.array_equal(cv_n[outs], r["conv"])
    assert np.array_equal(st_n[3], st[3].astype(np.float64))  # the checkpoint is untouched
    assert np.array_equal(cv_n[3], cv[3].astype(np.float64))


def test_decode_copy_on_write():
    """Requests 0 and 1 fork checkpoint row 2, request 2 forks row 4; they write rows 0, 5, 1.
    The checkpoints stay as they were, and each fork equals a decode step from its checkpoint."""
    import torch
    import gated_delta_rule_kda_amd as kda
    import oracle
    B, rows = 3, 6
    ins, outs = np.array([2, 2, 4], np.int32), np.array([0, 5, 1], np.int32)
    x = W.gen_decode(W.DecodeSpec(batch=B, heads=H, seed=65))
    st, cv = _pools(rows, 66)
    ro, rs, rc = oracle.decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], st[ins],
                                    g=x["g"], conv_w=x["conv_w"], conv_state=cv[ins])
    bf = torch.bfloat16
    st_d, cv_d = to_dev(st, torch.float32), to_dev(cv, bf)
    o = kda.decode_step(to_dev(x["q"], bf), to_dev(x["k"], bf), to_dev(x["v"], bf),
                        to_dev(x["log_alpha"], torch.float32), to_dev(x["beta"], torch.float32), st_d,
                        g=to_dev(x["g"], bf), conv_w=to_dev(x["conv_w"], torch.float32), conv_state=cv_d,
                        slots=to_dev(ins, torch.int32), slots_out=to_dev(outs, torch.int32), out_dtype="f32")
    torch.cuda.synchronize()
    st_n, cv_n = to_np(st_d), to_np(cv_d)
    assert err(to_np(o), ro) <= TOL["recurrent"]
    assert err(st_n[outs], rs) <= TOL["recurrent"]
    assert np.array_equal(cv_n[outs], rc)
    keep = [i for i in range(rows) if i not in outs]
    assert np.array_equal(st_n[keep], st[keep].astype(np.float64))
    assert np.array_equal(cv_n[keep], cv[keep].astype(np.float64))


def test_speculative_verify_then_replay():
    """Each of three requests proposes 5 draft tokens.  Verification runs them from the
    committed rows without writing anything; then the accepted prefixes (2, 5 and 0 tokens)
    are replayed in place, and one more decode step follows.  Everything equals the oracle
    run on the accepted token streams, and verification leaves the pools bit for bit."""
    import torch
    import gated_delta_rule_kda_amd as kda
    import oracle
    k_draft, acc = 5, [2, 5, 0]
    B, rows = 3, 8
    slots = [4, 1, 7]
    spec = W.PrefillSpec(lens=[k_draft + 1] * B, heads=H, seed=67)
    full = W.gen_prefill(spec)  # per request: 5 draft tokens, then the next decode token
    st, cv = _pools(rows, 68)
    st_d, cv_d = to_dev(st, torch.float32), to_dev(cv, torch.bfloat16)
    cu_full = full["cu_seqlens"].astype(np.int64)

    def take(tok_lists):
        tok = np.concatenate([np.asarray(t, np.int64) for t in tok_lists]) if tok_lists else np.zeros(0, np.int64)
        d = {n: full[n][tok] for n in ("q", "k", "v", "g", "log_alpha", "beta")}
        d["cu_seqlens"] = np.concatenate([[0], np.cumsum([len(t) for t in tok_lists])]).astype(np.int64)
        d["conv_w"] = full["conv_w"]
        return d

    drafts = take([np.arange(cu_full[n], cu_full[n] + k_draft) for n in range(B)])
    # 1. verify: read the committed rows, write nothing
    say("speculative: verify")
    o_ver = _dev_prefill(drafts, st_d, cv_d, "auto", slots, None, write=False)
    assert np.array_equal(to_np(st_d), st.astype(np.float64))
    assert np.array_equal(to_np(cv_d), cv.astype(np.float64))
    r_ver = oracle_prefill(dict(drafts, state_in=st[slots], conv_in=cv[slots]))
    assert err(o_ver, r_ver["o"]) <= TOL["auto"]
    # 2. replay the accepted prefixes in place
    say("speculative: replay")
    accepted = take([np.arange(cu_full[n], cu_full[n] + acc[n]) for n in range(B)])
    _dev_prefill(accepted, st_d, cv_d, "auto", slots, slots)
    r_acc = oracle_prefill(dict(accepted, state_in=st[slots], conv_in=cv[slots]))
    st_n, cv_n = to_np(st_d), to_np(cv_d)
    assert err(st_n[slots], r_acc["state"]) <= TOL["auto"]
    assert np.array_equal(cv_n[slots], r_acc["conv"])
    keep = [i for i in range(rows) if i not in slots]
    assert np.array_equal(st_n[keep], st[keep].astype(np.float64))
    # 3. one decode step per request continues from the replayed rows
    say("speculative: decode")
    nxt = np.array([cu_full[n] + acc[n] for n in range(B)])
    x = {n: full[n][nxt] for n in ("q", "k", "v", "g", "log_alpha", "beta")}
    bf = torch.bfloat16
    o = kda.decode_step(to_dev(x["q"], bf), to_dev(x["k"], bf), to_dev(x["v"], bf),
                        to_dev(x["log_alpha"], torch.float32), to_dev(x["beta"], torch.float32), st_d,
                        g=to_dev(x["g"], bf), conv_w=to_dev(full["conv_w"], torch.float32), conv_state=cv_d,
                        slots=to_dev(np.asarray(slots, np.int32), torch.int32), out_dtype="f32")
    torch.cuda.synchronize()
    ro, rs, rc = oracle.decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], r_acc["state"],
                                    g=x["g"], conv_w=full["conv_w"], conv_state=r_acc["conv"])
    assert err(to_np(o), ro) <= TOL["auto"]
    assert err(to_np(st_d)[slots], rs) <= TOL["auto"]
    assert np.array_equal(to_np(cv_d)[slots], rc)
