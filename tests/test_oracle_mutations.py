"""Each deliberate mistake planted in a copy of the oracle must fail at least
one pin.  The copies are built on the CPU with -DORC_PLANT=k (see oracle.c)
into a temporary directory; the real oracle is untouched."""
import pytest

import pins
from oracle import build

PLANTS = {
    1: "RoPE sine sign flipped",
    2: "GQA maps query head h to kv head h % n_kv",
    3: "attention scale 1/sqrt(d) dropped",
    4: "attention residual dropped",
    5: "gate and up swapped in SwiGLU",
    6: "RMSNorm gain dropped",
    7: "accept compares draft i with argmax i (off by one)",
    8: "cache advances by m instead of m+1",
    9: "n-gram matches the suffix itself",
    10: "argmax ties go to the highest index",
    11: "RoPE uses the row index instead of the position",
    12: "K rows of a span all written at the first position",
    13: "Philox round mixes the second key word into the first output word",
    14: "sampling multiplies the logits by the temperature instead of dividing",
    15: "a sliding-window row sees one key too many (window W + 1)",
    16: "the delta rule writes with the raw key instead of the unit key",
    17: "a partial accept keeps the recurrent state of the rejected rows",
}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda k: f"plant{k}")
def test_planted_mistake_is_caught(plant, tmp_path):
    lib = build.build(plant=plant, out=str(tmp_path / f"liboracle_plant{plant}.so"))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError as e:
            caught.append((pin.__name__, str(e)[:80]))
            break
        except Exception as e:  # an oracle error (e.g. NaN) also counts as caught
            caught.append((pin.__name__, repr(e)[:80]))
            break
    assert caught, f"no pin caught planted mistake {plant}: {PLANTS[plant]}"
