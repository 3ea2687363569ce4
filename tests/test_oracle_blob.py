"""Pins of the oracle's cache blob (codes saved with their scales): sizes
against the pages' per-cell byte counts, round trips, and refusal of blobs
whose layout facts differ (the pages' failure: int8 bytes restored without
their scales, or into a cache of another store type).

genie-ai-runtime release v0.1.0-alpha.11, "--int8-kv triage"; release
v0.1.0-alpha.12, "Path F (#45) interop guard"; Strata PR 2698, "What it does"
(528 B per int8 cell vs 2048 B for fp32 at head_dim 256)."""
import numpy as np
import pytest

from oracle import kvq_oracle as orc
import workloads as wl


def _cache(kdt="int8", vdt="int8", g=64, d=256, H=2, n=40, seed=81):
    c = orc.Cache(2, n, H, d, g, kdt, vdt)
    c.append(wl.uniform_rows(seed, (2, n, H, d)), wl.uniform_rows(seed + 1, (2, n, H, d)), [0, 0])
    return c


def test_payload_size_is_the_pages_cell_bytes():
    """Per position the int8 group-64 blob holds 528 B per store at head_dim
    256 with 2 kv heads (Strata's cell count), 2048 B per fp32 store."""
    for kdt, vdt, per_pos in (("int8", "int8", 2 * 528), ("int8", "fp32", 528 + 2048), ("fp32", "fp32", 4096)):
        c = _cache(kdt, vdt)
        n = 32  # a multiple of 16 positions: no region padding
        assert len(orc.blob_payload(c, 0, 0, n)) == n * per_pos
        assert per_pos == orc.cell_bytes(2, 256, 64, kdt) + orc.cell_bytes(2, 256, 64, vdt)


@pytest.mark.parametrize("kdt,vdt,g", [("int8", "int8", 64), ("int8", "int8", 256), ("int8", "fp32", 64),
                                       ("fp32", "int8", 64), ("fp32", "fp32", 64)])
def test_round_trip_restores_codes_and_scales(kdt, vdt, g):
    src = _cache(kdt, vdt, g)
    pay = orc.blob_payload(src, 1, 5, 23)
    hdr = orc.blob_header(src, 23)
    dst = orc.Cache(2, 40, 2, 256, g, kdt, vdt)
    orc.blob_restore(dst, hdr, pay, 0, 11)
    for s in ("k", "v"):
        np.testing.assert_array_equal(dst.data[s][0, 11:34], src.data[s][1, 5:28])
        if src.scales[s] is not None:
            np.testing.assert_array_equal(dst.scales[s][0, 11:34].view(np.uint16),
                                          src.scales[s][1, 5:28].view(np.uint16))
        # untouched elsewhere
        assert not dst.data[s][0, :11].any() and not dst.data[s][1].any()


def test_restored_cache_attends_like_the_original():
    src = _cache()
    dst = orc.Cache(1, 40, 2, 256, 64)
    orc.blob_restore(dst, orc.blob_header(src, 40), orc.blob_payload(src, 0, 0, 40), 0, 0)
    q = wl.uniform_rows(90, (2, 16, 256))
    want = orc.attend(q, src, [40, 40], 0, 1 / 16)[0]
    np.testing.assert_array_equal(orc.attend(q[:1], dst, [40], 0, 1 / 16)[0], want)


@pytest.mark.parametrize("field,value", [("k_dtype", 2), ("v_dtype", 2), ("scale_group", 256), ("head_dim", 128),
                                         ("n_kv_heads", 4), ("magic", 0), ("version", 2)])
def test_mismatched_blobs_are_refused(field, value):
    src = _cache()
    hdr = orc.blob_header(src, 8)
    hdr[field] = value
    with pytest.raises(ValueError):
        orc.blob_restore(orc.Cache(1, 40, 2, 256, 64), hdr, orc.blob_payload(src, 0, 0, 8), 0, 0)


def test_int8_payload_is_refused_by_an_fp32_cache_and_a_short_payload_too():
    src = _cache()
    with pytest.raises(ValueError):
        orc.blob_restore(orc.Cache(1, 40, 2, 256, 64, "fp32", "fp32"), orc.blob_header(src, 8),
                         orc.blob_payload(src, 0, 0, 8), 0, 0)
    with pytest.raises(ValueError):
        orc.blob_restore(orc.Cache(1, 40, 2, 256, 64), orc.blob_header(src, 8), orc.blob_payload(src, 0, 0, 8)[:-16],
                         0, 0)


# ---- 4-bit stores -----------------------------------------------------------------------

def test_q4_nibbles_unpack_to_their_codes():
    codes = np.random.default_rng(3).integers(0, 16, (5, 2, 256)).astype(np.uint8)
    np.testing.assert_array_equal(orc.unpack_q4(orc.pack_q4(codes)), codes)
    assert orc.unpack_q4(np.array([0xF0, 0xE1] + [0] * 14, dtype=np.uint8))[[0, 1, 16, 17]].tolist() == [0, 1, 15, 14]


def test_q4_payload_size_is_the_cell_bytes():
    """A q4 store's blob holds 128 code bytes and 8 fp16 scales per position
    and kv head (4.5 bits per value)."""
    for kdt, vdt in (("q4", "q4"), ("int8", "q4"), ("q4", "int8")):
        c = _cache(kdt, vdt)
        n = 32
        assert len(orc.blob_payload(c, 0, 0, n)) == n * (orc.cell_bytes(2, 256, 64, kdt) + orc.cell_bytes(2, 256, 64, vdt))
    assert orc.cell_bytes(2, 256, 64, "q4") == 2 * (128 + 16)


@pytest.mark.parametrize("kdt,vdt", [("q4", "q4"), ("int8", "q4"), ("q4", "int8")])
def test_q4_round_trip_and_attention_after_restore(kdt, vdt):
    src = _cache(kdt, vdt)
    pay = orc.blob_payload(src, 1, 3, 29)
    dst = orc.Cache(2, 40, 2, 256, 64, kdt, vdt)
    orc.blob_restore(dst, orc.blob_header(src, 29), pay, 0, 0)
    for s in ("k", "v"):
        np.testing.assert_array_equal(dst.data[s][0, :29], src.data[s][1, 3:32])
        np.testing.assert_array_equal(dst.scales[s][0, :29].view(np.uint16), src.scales[s][1, 3:32].view(np.uint16))
    q = wl.uniform_rows(91, (2, 16, 256))
    want = orc.attend(q, src, [32, 32], 0, 1 / 16)[1]
    # dst holds src's positions 3..31 of sequence 1 at 0..28; attend src over the same range via a window
    got = orc.attend(q[1:], dst, [29], 0, 1 / 16)[0]
    np.testing.assert_array_equal(got, orc.attend(q, src, [32, 32], 29, 1 / 16)[1])
    assert np.abs(got - want).max() > 0  # the window really changed the range


def test_q4_blob_is_refused_by_an_int8_cache():
    src = _cache("q4", "q4")
    hdr = orc.blob_header(src, 8)
    with pytest.raises(ValueError):
        orc.blob_restore(orc.Cache(1, 40, 2, 256, 64), hdr, orc.blob_payload(src, 0, 0, 8), 0, 0)
