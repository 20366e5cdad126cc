"""GPU: the offline reorder is exactly invertible and float32 dequantization is
bit-exact against the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import pack_canonical, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(16, 128, 0), (17, 256, 0), (1, 128, 0), (130, 384, 0), (256, 1024, 0),
          (48, 256, 1), (2 * 24, 128, 1), (4096, 7168, 1), (7168, 2048, 0)]


@pytest.mark.parametrize("N,K,flags", SHAPES)
def test_pack_unpack_round_trip(N, K, flags):
    import ffn_int4_g128_amd as q
    w = workloads.weights(21, N + K, N, K, 0.002, 0.02)
    packed = pack_canonical(w, flags)
    qw, sc, zr = q.unpack(packed, N, K, flags)
    assert np.array_equal(qw.cpu().numpy(), w["qweight"])
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), w["scales"])
    assert np.array_equal(zr.cpu().numpy(), w["zeros"])


@pytest.mark.parametrize("N,K,flags", SHAPES[:7])
def test_dequant_f32_bit_exact(N, K, flags):
    import ffn_int4_g128_amd as q
    w = workloads.weights(22, N * 3 + K, N, K, 0.002, 0.02)
    packed = pack_canonical(w, flags)
    got = q.dequant_f32(packed, N, K, flags).cpu().numpy()
    ref = oracle.dequant(w["qweight"], w["scales"], w["zeros"], N, K)
    assert np.array_equal(got.astype(np.float64), ref)


def test_pack_of_every_byte_value():
    """Each byte value at every position of a group survives the round trip."""
    import ffn_int4_g128_amd as q
    N, K = 32, 512
    qw = (np.arange(N * K // 2) % 256).astype(np.uint8).reshape(N, K // 2)
    qw = np.ascontiguousarray(np.roll(qw, 7, axis=1))
    sc = np.full((N, K // 128), 0x3C00, dtype=np.uint16)
    zr = (np.arange(N * K // 128) % 16).astype(np.uint8).reshape(N, K // 128)
    w = {"qweight": qw, "scales": sc, "zeros": zr, "N": N, "K": K}
    packed = pack_canonical(w)
    q2, s2, z2 = q.unpack(packed, N, K)
    assert np.array_equal(q2.cpu().numpy(), qw)
    assert np.array_equal(z2.cpu().numpy(), zr)
    got = q.dequant_f32(packed, N, K).cpu().numpy().astype(np.float64)
    assert np.array_equal(got, oracle.dequant(qw, sc, zr, N, K))
