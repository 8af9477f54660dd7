"""Host logic of the policies harness: the tables it writes from a saved run
(no GPU)."""
from emulated_fp32_matrix_amd import policies


def _run():
    pol = {}
    for name, mode, us in [("performant", "AUTO", (200.0, 190.0, 180.0)), ("native", "NATIVE_F32", (300.0, 290.0, 270.0))]:
        w, d, s = us
        pol[name] = {"mode": mode, "wall_us": w, "device_us": d, "steady_us": s,
                     "wall_tflops": 12.0 / w * 1e3, "device_tflops": 12.0 / d * 1e3, "steady_tflops": 12.0 / s * 1e3}
    return [{"stack": 2, "name": "stack two", "gflop": 12.0,
             "auto_choice": {"qkv.fwd": "BF16X9", "qkv.dX": "NATIVE_F32"},
             "auto_plan": {"qkv.fwd": [2, 128, 256], "qkv.dX": [1, 128, 96]}, "policies": pol}]


def test_policy_table_has_the_three_timings_and_speedups():
    md = policies._policy_markdown(_run())
    assert "| steady us | steady TFLOP/s | steady speedup |" in md
    row = [l for l in md.splitlines() if l.startswith("| performant |")][0].split("|")
    cells = [c.strip() for c in row[1:-1]]
    # wall, device and steady speedups are native time / policy time
    assert cells[4] == "1.50" and cells[7] == f"{290 / 190:.2f}" and cells[10] == "1.50"
    assert "qkv.fwd BF16X9 (S = 2 on the tiles from 256 on, 128-row tiles)" in md
    assert "qkv.dX NATIVE_F32," not in md and md.count("qkv.dX NATIVE_F32") == 1


def test_plan_text():
    assert policies._plan_text((1, 64, 96)) == "no split, 64-row tiles"
    assert policies._plan_text((4, 128, 0)) == "S = 4 on every tile, 128-row tiles"
    assert policies._plan_text((2, 128, 1024)) == "S = 2 on the tiles from 1024 on, 128-row tiles"
