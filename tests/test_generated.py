"""Generated sources are current: pv_asm.inc is exactly what gen_pv_asm.py writes."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_attention_compress_amd", "csrc")


def test_pv_asm_is_current():
    spec = importlib.util.spec_from_file_location("gen_pv_asm", os.path.join(CSRC, "gen_pv_asm.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    with open(os.path.join(CSRC, "pv_asm.inc")) as f:
        assert f.read() == gen.text()


def test_pv_asm_waits_cover_every_read():
    """Each MFMA's operand quad was filled by reads that its preceding lgkmcnt wait covers."""
    spec = importlib.util.spec_from_file_location("gen_pv_asm", os.path.join(CSRC, "gen_pv_asm.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    for ntiles in (1, 2):
        lines = [l.strip().strip('"').replace("\\n\\t", "").strip() for l in gen.block(ntiles).split("\\\n")]
        assert sum(l.startswith("v_mfma") for l in lines) == 32 * ntiles
        pending = []   # destination quads of issued, not yet waited reads (in order)
        for l in lines:
            if l.startswith("ds_read_b64_tr_b16"):
                reg = l.split()[1].rstrip(",")
                pending.append(int(reg[2:].split(":")[0]) & ~3)
            elif l.startswith("s_waitcnt lgkmcnt"):
                n = int(l.split("(")[1].rstrip(")"))
                pending = pending[len(pending) - n:] if n else []
            elif l.startswith("v_mfma"):
                quad = int(l.split()[2].rstrip(",")[2:].split(":")[0])
                assert quad not in pending, (ntiles, l)
