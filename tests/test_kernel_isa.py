"""Static checks of the attention kernels' gfx950 assembly, compiled here with the
library's own flags (no GPU needed).

An MFMA reads its A and B operands across all 64 lanes of the wave, so it must never
run while the exec mask is narrowed by a divergent branch: the inactive lanes' operand
rows would be dropped.  The compiler is free to move instructions whose results are only
used inside such a branch into it (it once moved the last tile's P^V MFMAs into the
epilogue's `row < N_q` branch), so every build is checked: a forward dataflow over each
kernel's control-flow graph marks where the mask may be narrowed (after
s_and_saveexec / s_or_saveexec, until exec is restored with s_or_b64 / s_mov_b64), and
no MFMA may be reachable in such a state.

The quantisers stage their input in LDS by global->LDS DMA (buffer_load ... lds), which
the hardware counts with the vector-memory counter, and nothing but an s_waitcnt on that
counter orders the DMA's LDS writes before the wave's own LDS reads: a read issued while
the DMA is in flight returns whatever the buffer held before (a fused K/V quantiser once
read partly landed chunks that way).  So every quantiser build is checked the same way:
no LDS read may be reachable while a DMA issued since the last vmcnt(0) may be in flight.
Each check is pinned by a synthetic listing that it must flag."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "mxfp4_bit_attention_amd"))


def _kernel_blocks(asm: str, name_re: str):
    """(symbol, basic blocks) of every kernel whose symbol matches name_re; a block is
    (label, [instructions])."""
    lines = asm.split("\n")
    starts = [k for k, l in enumerate(lines) if re.match(r"^" + name_re + r":", l)]
    for s in starts:
        # to the function's end label: the compiler may place blocks after s_endpgm
        e = next(k for k in range(s, len(lines)) if lines[k].startswith(".Lfunc_end"))
        blocks, cur = [], ("entry", [])
        for l in lines[s + 1:e]:
            t = l.strip()
            if not t or t.startswith(";"):
                continue
            m = re.match(r"^(\.LBB\d+_\d+):", t)
            if m:
                blocks.append(cur)
                cur = (m.group(1), [])
                continue
            if t.startswith("."):
                continue
            cur[1].append(t)
        blocks.append(cur)
        yield lines[s].split(":")[0], blocks


def _flagged(blocks, step) -> int:
    """Forward may-analysis of one boolean state over the control-flow graph (false at
    entry, OR at joins): step(instruction tokens, state) -> (new state, flagged).
    Returns the number of flagged instructions reachable in a flagging state."""
    idx = {b[0]: i for i, b in enumerate(blocks)}
    entry = [False] * len(blocks)

    def walk(i, mark):
        state, bad, fall = entry[i], 0, True
        for t in blocks[i][1]:
            tk = t.split()
            state, flag = step(tk, state)
            bad += flag
            if (tk[0].startswith("s_cbranch") or tk[0] == "s_branch") and tk[1] in idx:
                mark(idx[tk[1]], state)
            if tk[0] in ("s_branch", "s_endpgm"):
                fall = False
        if fall and i + 1 < len(blocks):
            mark(i + 1, state)
        return bad

    changed = [True]

    def mark(j, st):
        if st and not entry[j]:
            entry[j] = True
            changed[0] = True

    while changed[0]:
        changed[0] = False
        for i in range(len(blocks)):
            walk(i, mark)
    return sum(walk(i, lambda j, st: None) for i in range(len(blocks)))


def _mfma_step(tk, narrowed):
    op = tk[0]
    dst = tk[1].rstrip(",") if len(tk) > 1 else ""
    if op in ("s_and_saveexec_b64", "s_or_saveexec_b64"):
        narrowed = True
    elif op in ("s_or_b64", "s_mov_b64") and dst == "exec":
        narrowed = False
    return narrowed, int(op.startswith("v_mfma") and narrowed)


def mfma_under_narrowed_exec(asm: str) -> dict:
    """{kernel symbol: number of MFMAs reachable with a narrowed exec mask}."""
    return {name: _flagged(blocks, _mfma_step) for name, blocks in _kernel_blocks(asm, r"_Z\w*k_attn\w*")}


def _dma_step(tk, pending):
    op = tk[0]
    if op.startswith("buffer_load") and "lds" in tk:
        return True, 0
    if op == "s_waitcnt" and any(a.rstrip(",") == "vmcnt(0)" for a in tk[1:]):
        return False, 0
    return pending, int(op.startswith("ds_read") and pending)


def _lds_write_step(tk, pending):
    op = tk[0]
    if op.startswith("ds_write"):
        return True, 0
    if op == "s_waitcnt" and any(a.rstrip(",") == "lgkmcnt(0)" for a in tk[1:]):
        return False, 0
    return pending, int(op == "s_barrier" and pending)


def barrier_with_lds_write_in_flight(asm: str, name_re: str = r"_Z\w*k_(?:attn|quant)\w*") -> dict:
    """{kernel symbol: number of s_barrier reachable while an LDS write issued since the last
    lgkmcnt(0) wait may be in flight}.  s_barrier itself does not wait for the wave's
    memory operations on this part, so another wave may read LDS before such a write lands."""
    return {name: _flagged(blocks, _lds_write_step) for name, blocks in _kernel_blocks(asm, name_re)}


def lds_read_with_dma_in_flight(asm: str, name_re: str = r"_Z\w*k_quant\w*") -> dict:
    """{kernel symbol: number of LDS reads reachable while a global->LDS DMA issued since
    the last vmcnt(0) wait may still be in flight}."""
    return {name: _flagged(blocks, _dma_step) for name, blocks in _kernel_blocks(asm, name_re)}


def test_checker_flags_an_mfma_inside_a_divergent_branch():
    mfma = "  v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:19], v[20:23], v[0:15], v24, v25"
    asm = "\n".join([
        "_ZN6mxattn6k_attnILi128EEEvv:",
        "  v_cmp_gt_i32_e32 vcc, s0, v1",
        mfma,
        "  s_and_saveexec_b64 s[2:3], vcc",
        "  s_cbranch_execz .LBB0_2",
        ".LBB0_1:",
        mfma,                                   # under the narrowed mask
        "  global_store_dwordx4 v[30:31], v[0:3], off",
        "  s_cbranch_scc1 .LBB0_3",
        ".LBB0_2:",
        "  s_or_b64 exec, exec, s[2:3]",
        mfma,
        "  s_endpgm",
        ".LBB0_3:",                             # laid out after the program's end
        mfma,                                   # still under the narrowed mask
        "  s_branch .LBB0_2",
        ".Lfunc_end0:",
    ])
    assert list(mfma_under_narrowed_exec(asm).values()) == [2]


def _compile(tmp_path, name: str) -> str:
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    import build as b
    src = os.path.join(b.CSRC, name)
    out = str(tmp_path / (name + ".s"))
    cmd = [b.hipcc(), *b.common_flags(), *b.EXTRA_FLAGS.get(name, []), "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


def test_checker_flags_an_lds_read_racing_its_dma():
    dma, read = "  buffer_load_dwordx4 v1, s[4:7], 0 offen nt lds", "  ds_read_b128 v[2:5], v0"
    asm = "\n".join([
        "_ZN6mxattn16k_quant_hadamardILi128EEEvv:",
        dma,
        "  s_waitcnt vmcnt(0)",
        read,
        ".LBB0_1:",
        dma,
        read,                                   # the DMA just issued may be in flight
        "  s_waitcnt lgkmcnt(0)",
        "  s_cbranch_scc1 .LBB0_1",
        "  s_cbranch_scc0 .LBB0_2",
        "  s_waitcnt vmcnt(0)",
        read,
        "  s_endpgm",
        ".LBB0_2:",                             # laid out after the program's end
        read,                                   # reached with the loop's DMA in flight
        "  s_branch .LBB0_1",
        ".Lfunc_end0:",
    ])
    assert list(lds_read_with_dma_in_flight(asm).values()) == [2]


def test_no_quantiser_reads_lds_while_its_dma_may_be_in_flight(tmp_path):
    res = lds_read_with_dma_in_flight(_compile(tmp_path, "quantize.hip"))
    # Hadamard (d x input width x plain/error/arranged), token-axis and the fused K/V kernel
    assert sum("k_quant_hadamard" in k for k in res) == 12 and sum("k_quant_kv" in k for k in res) == 4
    assert all(n == 0 for n in res.values()), res
    # the bandwidth probe that reads its DMA'd LDS back (copy mode) obeys the same order
    probes = lds_read_with_dma_in_flight(_compile(tmp_path, "probes.hip"), r"_Z\w*k_stream_dma\w*")
    assert len(probes) == 2 and all(n == 0 for n in probes.values()), probes


def test_checker_flags_a_barrier_before_an_lds_write_lands():
    asm = "\n".join([
        "_ZN6mxattn6k_attnILi128EEEvv:",
        "  ds_write_b32 v0, v1",
        "  s_cbranch_scc1 .LBB0_2",
        "  s_waitcnt lgkmcnt(0)",
        "  s_barrier",
        ".LBB0_2:",
        "  s_barrier",                            # reached from the branch with the write in flight
        "  s_endpgm",
        ".Lfunc_end0:",
    ])
    assert list(barrier_with_lds_write_in_flight(asm).values()) == [1]


def test_no_barrier_passes_an_lds_write_in_flight(tmp_path):
    res = barrier_with_lds_write_in_flight(_compile(tmp_path, "attention.hip"))
    res.update(barrier_with_lds_write_in_flight(_compile(tmp_path, "quantize.hip")))
    assert sum("k_attn" in k for k in res) >= 8
    assert all(n == 0 for n in res.values()), res


def test_no_attention_mfma_runs_under_a_narrowed_exec_mask(tmp_path):
    res = mfma_under_narrowed_exec(_compile(tmp_path, "attention.hip"))
    assert len(res) >= 8  # every d x PNQ x dump x scale-layout instantiation
    assert all(n == 0 for n in res.values()), res
