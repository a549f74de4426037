"""The LDS race-check build (SGEMM_LDS_POISON=1) really poisons: its matrix
kernels write NaN into LDS ahead of the direct-to-LDS refills, which the
product build never does (its tiles fill LDS only by direct loads).  Checked
on the gfx950 assembly of mfma.hip, compiled here; no GPU needed."""
import concurrent.futures
import re

from dense_fp32_matrix_amd import build


def _counts(path):
    text = open(path).read()
    return {
        "dma": len(re.findall(r"^\s*global_load_lds_dword", text, flags=re.M)),
        "ds_write": len(re.findall(r"^\s*ds_write", text, flags=re.M)),
        "nan": len(re.findall(r"0x7fc00000", text)),
    }


def test_poison_build_writes_nan_before_refills(tmp_path):
    plain = tmp_path / "mfma.s"
    poison = tmp_path / "mfma_poison.s"
    with concurrent.futures.ThreadPoolExecutor(2) as ex:
        jobs = [ex.submit(build.asm, "mfma.hip", str(plain)),
                ex.submit(build.asm, "mfma.hip", str(poison), lds_poison=True)]
        for j in jobs:
            j.result()
    p, q = _counts(plain), _counts(poison)
    assert p["dma"] > 0 and p["dma"] == q["dma"]
    assert p["ds_write"] == 0 and p["nan"] == 0
    # one poison store per direct load (the compiler may pair 4-byte ones)
    assert q["ds_write"] >= q["dma"] // 2 and q["nan"] > 0
