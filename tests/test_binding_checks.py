"""The Python binding refuses mismatched buffers before anything reaches the library.

The kernels index every buffer as the dense shape the C ABI describes, so a tensor of the
wrong shape, dtype or layout would be read or written out of bounds. These host-only tests
hand the binding tensors that claim to be device tensors (a subclass reporting
``is_cuda``) and check that each mismatch raises ``ValueError`` while the library is never
touched (its loader is replaced by one that fails the test). A valid call of each kind
reaches the loader, so the checks do not simply reject everything.
"""

import pytest
import torch

import draft_tree_verification_tv_amd.tv as tvb

N, HQ, HKV, D, L = 4, 8, 2, 128, 16


class FakeDev(torch.Tensor):
    """A host tensor that the binding's device checks accept."""

    @property
    def is_cuda(self):
        return True


def fd(t):
    return torch.Tensor._make_subclass(FakeDev, t)


class Reached(Exception):
    pass


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def _lib():
        raise Reached("library reached")
    monkeypatch.setattr(tvb, "lib", _lib)


def bf(*shape):
    return fd(torch.zeros(shape, dtype=torch.bfloat16))


def i32(*shape):
    return fd(torch.zeros(shape, dtype=torch.int32))


def f32(*shape):
    return fd(torch.zeros(shape, dtype=torch.float32))


def attn_args(**kw):
    a = dict(q=bf(N, HQ, D), k=bf(L + N, HKV, D), v=bf(L + N, HKV, D), parent=i32(N), L=L,
             workspace=fd(torch.zeros(1 << 16, dtype=torch.uint8)))
    a.update(kw)
    return a


def call_attn(a):
    return tvb.tree_attn(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("parent"), **a)


def test_tree_attn_valid_call_reaches_the_library():
    with pytest.raises(Reached):
        call_attn(attn_args())


@pytest.mark.parametrize("label,kw", [
    ("k head dim", dict(k=bf(L + N, HKV, 64))),
    ("v head dim", dict(v=bf(L + N, HKV, 64))),
    ("v heads", dict(v=bf(L + N, HKV + 1, D), k=bf(L + N, HKV + 1, D)[:, :HKV])),
    ("k/v heads differ", dict(v=bf(L + N, 1, D).expand(L + N, HKV, D))),
    ("parent length", dict(parent=i32(N + 1))),
    ("parent dtype", dict(parent=fd(torch.zeros(N, dtype=torch.int64)))),
    ("parent strided", dict(parent=i32(2 * N)[::2])),
    ("out shape", dict(out=bf(N, HQ, D + 8))),
    ("out dtype", dict(out=f32(N, HQ, D))),
    ("out strided", dict(out=bf(N, HQ, 2 * D)[:, :, :D])),
    ("lse shape", dict(lse=f32(N, HQ + 1))),
    ("lse dtype", dict(lse=bf(N, HQ))),
    ("lse strided", dict(lse=f32(HQ, N).t())),
    ("dev_error dtype", dict(dev_error=f32(1))),
    ("short cache", dict(L=L + 1)),
    ("workspace strided", dict(workspace=fd(torch.zeros(1 << 17, dtype=torch.uint8))[::2])),
])
def test_tree_attn_rejects(label, kw):
    with pytest.raises(ValueError):
        call_attn(attn_args(**kw))


def fp8_args(**kw):
    codes = fd(torch.zeros((L + N, HKV, D), dtype=torch.uint8))
    a = dict(q=bf(N, HQ, D), k_codes=codes, v_codes=fd(torch.zeros((L + N, HKV, D), dtype=torch.uint8)),
             k_exps=i32(L + N, HKV), v_exps=i32(L + N, HKV), parent=i32(N), L=L,
             workspace=fd(torch.zeros(1 << 16, dtype=torch.uint8)))
    a.update(kw)
    return a


def call_fp8(a):
    return tvb.tree_attn_fp8(a.pop("q"), a.pop("k_codes"), a.pop("v_codes"), a.pop("k_exps"), a.pop("v_exps"),
                             a.pop("parent"), **a)


def test_tree_attn_fp8_valid_call_reaches_the_library():
    with pytest.raises(Reached):
        call_fp8(fp8_args())


@pytest.mark.parametrize("label,kw", [
    ("code head dim", dict(k_codes=fd(torch.zeros((L + N, HKV, 64), dtype=torch.uint8)),
                           v_codes=fd(torch.zeros((L + N, HKV, 64), dtype=torch.uint8)))),
    ("v exps heads", dict(v_exps=i32(L + N, HKV + 1))),
    ("parent length", dict(parent=i32(N - 1))),
    ("out shape", dict(out=bf(N + 1, HQ, D))),
    ("lse shape", dict(lse=f32(N, HQ, 1))),
])
def test_tree_attn_fp8_rejects(label, kw):
    with pytest.raises(ValueError):
        call_fp8(fp8_args(**kw))


def test_accept_checks():
    parent, draft, tok = i32(N), i32(N), i32(N)
    with pytest.raises(Reached):
        tvb.accept(parent, draft, tok)
    for bad in (dict(draft=i32(N - 1)), dict(tok=i32(N + 1)), dict(tok=i32(2 * N)[::2])):
        a = dict(parent=parent, draft=draft, tok=tok)
        a.update(bad)
        with pytest.raises(ValueError):
            tvb.accept(a["parent"], a["draft"], a["tok"])
    short = (i32(1), i32(N - 1), i32(N), i32(1))
    with pytest.raises(ValueError):
        tvb.accept(parent, draft, tok, out=short)
    with pytest.raises(ValueError):
        tvb.accept(parent, draft, tok, out=(i32(1), i32(N), i32(N)))


def test_argmax_checks():
    V = 100
    lg = bf(N, V)
    ws = fd(torch.zeros(4096, dtype=torch.uint8))
    with pytest.raises(Reached):
        tvb.argmax(lg, workspace=ws)
    with pytest.raises(Reached):
        tvb.argmax(lg, V=V - 3, workspace=ws)
    for bad in (dict(V=V + 1), dict(V=0), dict(tok=i32(N - 1)), dict(tok=f32(N))):
        with pytest.raises(ValueError):
            tvb.argmax(lg, workspace=ws, **bad)


@pytest.mark.parametrize("fn", ["argmax_accept", "sample_accept"])
def test_argmax_accept_checks(fn):
    V = 100
    lg = bf(N, V)
    ws = fd(torch.zeros(4096, dtype=torch.uint8))
    extra = (1.0, 7) if fn == "sample_accept" else ()
    call = getattr(tvb, fn)
    with pytest.raises(Reached):
        call(lg, i32(N), i32(N), *extra, workspace=ws)
    bads = [dict(parent=i32(N + 1)), dict(draft=i32(N - 1)), dict(V=V + 1), dict(tok=i32(N + 2)),
            dict(out=(i32(1), i32(N - 1), i32(N), i32(1)))]
    for bad in bads:
        a = dict(parent=i32(N), draft=i32(N))
        a.update(bad)
        p, d = a.pop("parent"), a.pop("draft")
        with pytest.raises(ValueError):
            call(lg, p, d, *extra, workspace=ws, **a)


def test_kv_commit_checks():
    k, v = bf(L + N, HKV, D), bf(L + N, HKV, D)
    with pytest.raises(Reached):
        tvb.kv_commit(k, v, L, i32(1), i32(N))
    with pytest.raises(ValueError):
        tvb.kv_commit(k, v, L, i32(1), i32(N), N=N + 1)       # more nodes than accept_nodes holds
    with pytest.raises(ValueError):
        tvb.kv_commit(k, v, L, f32(1), i32(N))
    with pytest.raises(ValueError):
        tvb.kv_commit(k, v, L + 1, i32(1), i32(N))            # cache too short
    with pytest.raises(ValueError):
        tvb.kv_commit(k, v, L, i32(1), i32(N), new_len=f32(1))
