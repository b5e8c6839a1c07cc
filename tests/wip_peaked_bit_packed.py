"""Peaked-softmax parity of the bit-packed layout (work in progress: its key path still rounds to fp16)."""
from test_gpu_peaked import *  # noqa: F401,F403

PACKED = [(R, L, s, pl) for R in (11, 21) for L in (8192, 131072) for s, pl in
          ((3, False), (6, False), (12, False), (3, True), (12, True))]


@pytest.mark.parametrize("R,L,score_std,planted", PACKED)
def test_peaked_bit_packed(vq, R, L, score_std, planted):
    kw = dict(n_residuals=R)
    name = f"peak_g64_r{R}_{L}_s{score_std}{'_pl' if planted else ''}"
    announce(f"{name}")
    cfg = workloads.custom(name, 1, 32, 8, (L,), R, "float16", 500 + R + score_std + (50 if planted else 0),
                           n_groups=2, n_codes=64, q_std=q_std_for(score_std, kw))
    inp = workloads.make_inputs(cfg)
    if planted:
        inp = plant(cfg, inp, plant_positions(L))
    got, ref = run_case(vq, cfg, inp)
    err = rowwise_rel_err(got, ref)
    print(f"{name}: max row-relative error {err:.3e} (tol {TOL['float16']})", flush=True)
    assert err <= TOL["float16"]




def test_peaked_ragged_bit_packed(vq):
    kw = dict(n_residuals=11)
    name = "peak_ragged_bit_packed_r11"
    announce(name)
    base = workloads.Config(name, 16, 32, 8, None, 11, "float16", 611, ragged_range=(4096, 65536),
                            q_std=q_std_for(6, kw), n_groups=2, n_codes=64)
    inp = workloads.make_inputs(base)
    lens = [int(x) for x in inp["seq_len"]]
    inp = plant(base, inp, [(b, (977 * b + 131) % lens[b], (3 * b) % 32) for b in range(16)])
    got, ref = run_case(vq, base, inp)
    err = rowwise_rel_err(got, ref)
    print(f"{name}: max row-relative error {err:.3e} (tol {TOL['float16']})", flush=True)
    assert err <= TOL["float16"]
