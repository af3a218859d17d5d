"""The matrix-phase asm of the ping-pong bf16 forward is generated text
(exact_attention_28_amd/csrc/fa_pp_asm.h, written by gen_pp_asm.py beside
it). These checks keep the committed header identical to what the generator
writes, and check the generated sequence itself: every product waits for
its own LDS reads and for nothing issued after them, no fragment slot is
overwritten before the product that reads it has been issued, and the
offsets stay inside one LDS tile buffer."""
import importlib.util
import os
import re

CSRC = os.path.join(os.path.dirname(__file__), "..", "exact_attention_28_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_pp_asm", os.path.join(CSRC, "gen_pp_asm.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_header_matches_generator(tmp_path):
    g = _gen()
    with open(os.path.join(CSRC, "fa_pp_asm.h")) as f:
        committed = f.read()
    for which, name in (("both", "PP_ASM_BOTH"), ("s", "PP_ASM_S"), ("pv", "PP_ASM_PV")):
        for ins in g.block(which):
            assert f'"{ins}\\n\\t"' in committed, (name, ins)
    # the header holds nothing else than the three blocks
    n = sum(len(g.block(w)) for w in ("both", "s", "pv"))
    assert committed.count('\\n\\t"') == n


def _simulate(lines):
    """Walk a generated block and return its products in order, checking
    that each product's A operand has landed (no read into its registers
    still counted in flight) and that a fragment slot is refilled only
    after the product reading the previous fill was issued."""
    inflight = []   # register ranges of issued reads, oldest first
    pending = set() # registers filled by a read and not yet read by a product
    products = []
    for ins in lines:
        m = re.match(r"ds_read_\S+ v\[(\d+):(\d+)\], %\[(ka|va)\] offset:(\d+)", ins)
        if m:
            lo, hi, off = int(m.group(1)), int(m.group(2)), int(m.group(4))
            regs = set(range(lo, hi + 1))
            assert not (regs & pending), ins
            pending |= regs
            inflight.append(regs)
            assert off + len(regs) * 4 <= 16640, ins
            continue
        m = re.match(r"s_waitcnt lgkmcnt\((\d+)\)", ins)
        if m:
            while len(inflight) > int(m.group(1)):
                inflight.pop(0)
            continue
        m = re.match(r"v_mfma_f32_32x32x16_bf16 \S+, v\[(\d+):(\d+)\]", ins)
        if m:
            regs = set(range(int(m.group(1)), int(m.group(2)) + 1))
            assert all(not (regs & r) for r in inflight), ins
            assert regs <= pending, ins
            pending -= regs
            products.append(ins)
    assert not inflight and not pending
    return products


def test_generated_sequence_waits_and_slots():
    g = _gen()
    for which, n in (("both", 32), ("s", 16), ("pv", 16)):
        prods = _simulate(g.block(which))
        assert len(prods) == n
        # score chains start from zero, products accumulate in place
        for p in prods:
            dst = p.split()[1].rstrip(",")
            src_c = p.split()[-1]
            assert src_c in ("0", dst)
