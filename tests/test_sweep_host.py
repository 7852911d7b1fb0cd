"""Host-side checks of the length sweep's geometry (no GPU): its density and
flop counts agree with the oracle's mask on the same layouts."""
import pytest

from oracle import vdn_oracle as O
from video_diffusion_hybrid_block_amd import sweep as S


@pytest.mark.parametrize("T", [1, 2, 7, 42, 60, 81, 102])
@pytest.mark.parametrize("C,W", [(5, 1), (3, 2), (2, 0)])
def test_density_matches_oracle(T, C, W):
    lay = O.Layout(batch=1, heads=1, head_dim=16, frames=T, tokens_per_frame=4, text_tokens=0,
                   chunk_frames=C, window_chunks=W)
    assert S.density(T, C, W, True) == pytest.approx(O.softmax_density(lay, True), abs=1e-12)
    assert S.density(T, C, W, False) == pytest.approx(O.softmax_density(lay, False), abs=1e-12)


def test_dense_window_is_full_attention():
    T, P, L, H, d = 11, 8, 3, 2, 16
    nc = (T + 4) // 5
    assert S.density(T, 5, nc) == 1.0
    assert S.softmax_flops(T, P, L, H, d, 5, nc) == 4.0 * d * (T * P) * (T * P + L) * H


def test_anchor_increment_at_102_frames():
    # the pages print +3.57 % (tests/golden/anchor_density.txt)
    inc = 100 * (S.density(102) - S.density(102, anchors=False))
    assert int(inc * 100) / 100 == 3.57


def _tiles_brute(lay, text):
    """Per query frame, the oracle's visible key tokens packed back to back
    (window and anchor frames, then the text), cut into 64-key tiles one tile
    at a time; every frame has ceil(P / 256) query items."""
    P, L = lay.tokens_per_frame, lay.text_tokens
    items = len(range(0, P, 256))
    total = 0
    for t in range(lay.frames):
        keys = [f * P + i for f in O.visible_frames(lay, t) for i in range(P)]
        if text:
            keys += [lay.frames * P + j for j in range(L)]
        n_tiles = 0
        while keys:
            keys = keys[64:]
            n_tiles += 1
        total += items * n_tiles
    return total


@pytest.mark.parametrize("T,P,L,C,W", [(7, 100, 30, 2, 1), (12, 300, 0, 5, 1), (9, 64, 17, 3, 0),
                                       (1, 257, 5, 5, 1)])
@pytest.mark.parametrize("text", [False, True])
def test_tile_count_matches_oracle_mask(T, P, L, C, W, text):
    lay = O.Layout(batch=1, heads=1, head_dim=16, frames=T, tokens_per_frame=P, text_tokens=L,
                   chunk_frames=C, window_chunks=W)
    assert S.tile_count(T, P, L, C, W, True, text) == _tiles_brute(lay, text)


@pytest.mark.parametrize("T", [42, 102])
def test_tile_density_equals_frame_density_on_whole_tiles(T):
    # 1024 tokens per frame: every frame is 16 whole key tiles and 4 whole
    # query items, so tile and frame-pair densities coincide exactly
    assert S.tile_density(T, 1024, 0) == pytest.approx(S.density(T), abs=1e-15)
    inc_t = S.tile_density(T, 1024, 0) - S.tile_density(T, 1024, 0, anchors=False)
    assert inc_t == pytest.approx(S.density(T) - S.density(T, anchors=False), abs=1e-15)


def test_tile_rows_768p_frames():
    rows = {r["frames"]: r for r in S.tile_rows([42, 102])}
    # at the 1008-token frame the partial tiles move the density by less than
    # 0.05 points and the anchors' increment by less than 0.1
    for r in rows.values():
        assert abs(r["tile_density_pct"] - r["density_pct"]) < 0.05
        assert abs(r["tile_anchor_increment_pct"] - r["anchor_increment_pct"]) < 0.1
