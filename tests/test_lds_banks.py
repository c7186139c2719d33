"""LDS bank model of gfx950 and the swizzles of the bf16 kernels (CPU only).

Model: 64 banks of 4 bytes.  ds_read_b128 serves 16 lanes per cycle, lanes
8a .. 8a+7 together with 32+8a .. 32+8a+7; ds_read_b64_tr_b16 serves lanes
0..31, then 32..63.  A cycle costs as many passes as the most-used bank has
distinct words.  With this grouping the model gives the conflict counts the
SQ_LDS_BANK_CONFLICT counter measured on the kernels: none for the forward
loop kernel and the backward weight kernel, and for the backward token kernel
with its earlier hidden-unit swizzle exactly 4 extra cycles per row-fragment
read (2048 wavefronts x 768 reads x 4 = 6.29e6 per launch).

Each address formula below restates the one in the kernel source named in its
docstring; the tests check that every read pattern costs the ideal number of
cycles (4 for b128, 2 for the transpose read)."""
import pytest

ROWB = 256


def groups_b128():
    return [[l for l in range(64) if (l >> 3) & 3 == a] for a in range(4)]


def groups_tr():
    return [list(range(32)), list(range(32, 64))]


def cycles(addrs, nbytes, groups):
    total = 0
    for grp in groups:
        banks = {}
        for lane in grp:
            for w in range(addrs[lane] // 4, (addrs[lane] + nbytes) // 4):
                banks.setdefault(w % 64, set()).add(w)
        total += max(len(v) for v in banks.values())
    return total


def swz4(t):  # swiglu_loop.hip
    return (t & 1) | ((t & 6) << 1) | ((t & 8) >> 2)


def swz_u(t):  # swiglu_bwd.hip, hidden-unit stage
    return ((t & 7) << 1) | (t & 1)


def swz_u_previous(t):
    return ((t & 7) << 1) | ((t >> 3) & 1)


def swz_t(t):  # swiglu_bwd.hip, token stage
    return ((t & 3) << 1) | (t & 8) | ((t >> 2) & 1)


def loop_grad_rows(kk, ti):
    """Forward loop kernel, gradient wave: K / V row fragments."""
    return [(16 * ti + (l & 15)) * ROWB + 16 * ((4 * kk + (l >> 4)) ^ swz4(l & 15)) for l in range(64)]


def loop_state_tr(t, odd, half):
    """Forward loop kernel, state wave: K^T / V^T transpose fragments."""
    out = []
    for l in range(64):
        p, g = l & 15, l >> 4
        q, r0 = p & 3, 4 * g + (p >> 2)
        h0 = 8 * (q & 1)
        a = r0 * ROWB + 16 * ((4 * t + q) ^ swz4(r0)) + h0
        out.append(a + (8 - 2 * h0 if odd else 0) + 4096 * half)
    return out


def tok_afrag(kk, swz):
    """Backward token kernel: projection A fragments (b128)."""
    return [(l & 15) * ROWB + 16 * ((4 * kk + (l >> 4)) ^ swz(l & 15)) for l in range(64)]


def tok_tr_units(n, swz):
    """Backward token kernel: hidden-major B fragments (transpose read)."""
    out = []
    for l in range(64):
        p, g = l & 15, l >> 4
        row, q = 4 * g + (p >> 2), p & 3
        out.append(row * ROWB + 16 * ((2 * n + (q >> 1)) ^ swz(row)) + 8 * (q & 1))
    return out


def wt_tr_tokens(n, h):
    """Backward weight kernel: token-major B fragments (transpose read)."""
    out = []
    for l in range(64):
        p, g = l & 15, l >> 4
        q, row = p & 3, 8 * g + 4 * h + (p >> 2)
        out.append(row * ROWB + 16 * ((2 * n + (q >> 1)) ^ swz_t(row & 15)) + 8 * (q & 1))
    return out


@pytest.mark.parametrize("kk", range(4))
@pytest.mark.parametrize("ti", range(2))
def test_forward_row_fragments(kk, ti):
    assert cycles(loop_grad_rows(kk, ti), 16, groups_b128()) == 4


@pytest.mark.parametrize("t", range(4))
@pytest.mark.parametrize("odd", [0, 1])
@pytest.mark.parametrize("half", [0, 1])
def test_forward_transpose_fragments(t, odd, half):
    assert cycles(loop_state_tr(t, odd, half), 8, groups_tr()) == 2


@pytest.mark.parametrize("kk", range(4))
def test_backward_token_row_fragments(kk):
    assert cycles(tok_afrag(kk, swz_u), 16, groups_b128()) == 4
    # the earlier swizzle: the 2-way conflict the counter measured
    assert cycles(tok_afrag(kk, swz_u_previous), 16, groups_b128()) == 8


@pytest.mark.parametrize("n", range(8))
def test_backward_token_transpose_fragments(n):
    assert cycles(tok_tr_units(n, swz_u), 8, groups_tr()) == 2


@pytest.mark.parametrize("n", range(8))
@pytest.mark.parametrize("h", range(2))
def test_backward_weight_transpose_fragments(n, h):
    assert cycles(wt_tr_tokens(n, h), 8, groups_tr()) == 2


def test_swizzles_stay_in_row():
    for swz in (swz4, swz_u, swz_t):
        assert all(0 <= swz(t) < 16 for t in range(16))
