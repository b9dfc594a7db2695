"""Full-size parity, LongCat/DeepSeek-class routed-expert layer: d=7168,
f=2048, 256 experts, top-8 renormalised, e4m3 with 128x128 f32 scales
(11.3 GB of expert weights), at 1, 64 and 4096 tokens on both expert paths
and with quantised activations.  Every token and every slot is compared with
the oracle: routing bit for bit, h within one bf16 step, out within the
output bars."""
import pytest

from full_size import FullSize

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def full():
    f = FullSize("large-e4m3").setup()
    yield f
    f.teardown()


@pytest.mark.parametrize("T,path", [(1, 0), (1, 2), (64, 0), (64, 2), (4096, 0)])
def test_large_e4m3(full, T, path):
    full.check(T, path)


@pytest.mark.parametrize("T", [512])
def test_large_e4m3_act_quant(full, T):
    full.check_act_quant(T)
