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
