"""CPU checks of the seeded input generators (no attention arithmetic here)."""
import numpy as np
import pytest

from exact_attention_88_amd import workloads as W


def test_bf16_rounding_matches_round_to_nearest_even():
    """round_to_bf16 gives the nearest bfloat16 value, ties to even, as an
    independent bit-level rule and torch's CPU cast both say."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(37.0)
    # exact ties: the low 16 bits are 0x8000, for even and odd kept halves
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], dtype=np.uint32)
    x = np.concatenate([x, ties.view(np.float32)])
    r = W.round_to_bf16(x)
    ru = r.view(np.uint32)
    assert np.all((ru & 0xFFFF) == 0)
    # nearest: |x - r| <= half an ulp of bfloat16 at r
    ulp = np.abs(np.spacing(r.astype(np.float32)).astype(np.float64)) * 65536
    assert np.all(np.abs(x.astype(np.float64) - r.astype(np.float64)) <= ulp / 2 + 1e-30)
    # ties go to the even kept half
    rt = W.round_to_bf16(ties.view(np.float32)).view(np.uint32)
    assert np.all(((rt >> 16) & 1) == 0)
    torch = pytest.importorskip("torch")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ref.view(np.uint32), ru)


def test_bf16_case_inputs_are_bf16_values():
    case = W.bf16_cases()[0]
    x = W.make_inputs(case)
    for name, a in x.items():
        bits = np.ascontiguousarray(a).view(np.uint32)
        assert np.all((bits & 0xFFFF) == 0), name
        assert a.shape == ((case.B, case.H, case.Sq if name in ("q", "do") else case.Sk, case.D))
