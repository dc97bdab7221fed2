"""MI355X-native DSpark sequential Markov draft-sampling step.

A thin ctypes binding over ``libmarkov.so`` (HIP kernels for gfx950 behind
the C ABI in ``include/markov.h``). The functions here marshal arguments
only: every step of the computation runs in the library's kernels, and the
binding raises if the library is missing -- there is no CPU path.

PyTorch serves for device memory and streams: tensors are passed by
``data_ptr()`` and the stream defaults to torch's current stream.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libmarkov.so")

OK = 0
ERRORS = {
    -1: "MARKOV_ERR_NULL", -2: "MARKOV_ERR_SHAPE", -3: "MARKOV_ERR_RANK",
    -4: "MARKOV_ERR_ALIGN", -5: "MARKOV_ERR_ROWS", -6: "MARKOV_ERR_WORKSPACE",
    -7: "MARKOV_ERR_HIP", -8: "MARKOV_ERR_VOCAB",
}


class MarkovError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        name = ERRORS.get(status, str(status))
        super().__init__(f"{what}: {name} ({status_string(status)})" if what else name)


class Shape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("vocab", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("mult", ctypes.c_float), ("softcap", ctypes.c_float)]


_P = ctypes.c_void_p
_SIGS = {
    "markov_max_rows": (ctypes.c_int32, [ctypes.c_int32]),
    "markov_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32]),
    "markov_workspace_init": (ctypes.c_int, [_P, ctypes.c_size_t, ctypes.POINTER(Shape), _P]),
    "markov_why_not": (ctypes.c_char_p, [ctypes.POINTER(Shape), ctypes.c_int32]),
    "markov_sample_sequential": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P,
                                                _P, _P, ctypes.POINTER(Shape), _P,
                                                ctypes.c_size_t]),
    "markov_debug_sample_exact": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P,
                                                 _P, _P, ctypes.POINTER(Shape), _P,
                                                 ctypes.c_size_t]),
    "markov_debug_sample_fallback": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int32, _P,
                                                    _P, _P, _P, ctypes.POINTER(Shape), _P,
                                                    ctypes.c_size_t]),
    "markov_sample_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                          _P, _P, _P, _P, ctypes.POINTER(Shape), _P,
                                          ctypes.c_size_t]),
    "markov_sample_sequential_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                                        _P, _P, _P, _P, ctypes.POINTER(Shape)]),
    "markov_noalloc_max_rows": (ctypes.c_int32, []),
    "markov_greedy_sequential": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P,
                                                ctypes.POINTER(Shape), _P, ctypes.c_size_t]),
    "markov_greedy_step": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                          _P, _P, ctypes.POINTER(Shape), _P, ctypes.c_size_t]),
    "markov_greedy_finalize": (ctypes.c_int, [_P, ctypes.c_int64, _P, _P]),
    "markov_quantize_w2_fp8": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P]),
    "markov_sample_sequential_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                                    _P, _P, _P, _P, ctypes.POINTER(Shape), _P,
                                                    ctypes.c_size_t]),
    "markov_greedy_sequential_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int32, _P, _P,
                                                    _P, _P, ctypes.POINTER(Shape), _P,
                                                    ctypes.c_size_t]),
    "markov_debug_e4m3_encode": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "markov_debug_e4m3_decode": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "markov_shard_step": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, _P, _P, ctypes.c_int32,
                                         ctypes.c_int32, _P, _P, _P, ctypes.c_int32,
                                         ctypes.c_int32, _P, ctypes.POINTER(Shape), _P,
                                         ctypes.c_size_t]),
    "markov_pick": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, _P, _P]),
    "markov_verify_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "markov_greedy_accept": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, _P, _P, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t, _P]),
    "markov_prob_accept": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P,
                                          ctypes.c_size_t, _P]),
    "markov_debug_bias_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.POINTER(Shape), _P]),
    "markov_sample_step_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                              ctypes.c_int32, _P, _P, _P, _P,
                                              ctypes.POINTER(Shape), _P, ctypes.c_size_t]),
    "markov_greedy_step_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                              _P, _P, _P, _P, ctypes.POINTER(Shape), _P,
                                              ctypes.c_size_t]),
    "markov_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "markov_debug_bias": (ctypes.c_int, [_P, _P, _P, _P, ctypes.POINTER(Shape), _P]),
    "markov_debug_gumbel": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_float,
                                           ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, _P,
                                           _P, _P, _P]),
    "markov_debug_bf16_round": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "markov_debug_copy": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "markov_debug_noise_table": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "markov_debug_transform_table": (ctypes.c_int32, [ctypes.c_float, ctypes.c_float, _P,
                                                      ctypes.c_int32]),
}

_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(
                f"{LIBRARY} is missing: build it first (python -c 'import __graft_entry__ as g; "
                "g.build()'); there is no CPU fallback")
        handle = ctypes.CDLL(LIBRARY)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().markov_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != OK:
        raise MarkovError(status, what)


def make_shape(rows: int, vocab: int, rank: int, mult: float = 1.0, softcap: float = 0.0):
    return Shape(int(rows), int(vocab), int(rank), float(mult), float(softcap))


def max_rows(rank: int) -> int:
    return int(lib().markov_max_rows(int(rank)))


def workspace_bytes(rows: int, vocab: int, rank: int, k: int, mult: float = 1.0,
                    softcap: float = 0.0) -> int:
    sh = make_shape(rows, vocab, rank, mult, softcap)
    return int(lib().markov_workspace_bytes(ctypes.byref(sh), int(k)))


def why_not(rows: int, vocab: int, rank: int, k: int, mult: float = 1.0,
            softcap: float = 0.0) -> str | None:
    sh = make_shape(rows, vocab, rank, mult, softcap)
    r = lib().markov_why_not(ctypes.byref(sh), int(k))
    return None if r is None else r.decode()


# -- tensors ---------------------------------------------------------------------

def _stream_ptr(stream):
    if stream is None:
        import torch

        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name, shape=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def new_workspace(rows: int, vocab: int, rank: int, k: int, device="cuda", stream=None,
                  mult: float = 1.0, softcap: float = 0.0):
    """Allocate and prepare a workspace for this shape (a uint8 tensor); the
    output-transform table in it is built for (mult, softcap)."""
    import torch

    sh = make_shape(rows, vocab, rank, mult, softcap)
    n = workspace_bytes(rows, vocab, rank, k)
    if n == 0:
        raise MarkovError(-2, "workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check(lib().markov_workspace_init(ctypes.c_void_p(ws.data_ptr()), n, ctypes.byref(sh),
                                       _stream_ptr(stream)),
           "markov_workspace_init")
    return ws


def sample_sequential(base_logits, w1, w2, prev, seeds, positions, temperature, cache, tokens,
                      workspace, mult: float = 1.0, softcap: float = 0.0, stream=None,
                      exact: bool = False, step: int | None = None, fallback: bool = False):
    """markov_sample_sequential: base_logits/cache bf16 [rows, k, V], w1/w2 bf16
    [V, R], prev/seeds int64 [rows], positions/tokens int64 [rows, k],
    temperature fp32 [rows], workspace from ``new_workspace``. ``exact`` runs
    the test-only variant that takes the exact key at every element,
    ``fallback`` the one that sends every noisy row through the exact re-read
    path; ``step`` runs that one step of the loop alone (markov_sample_step)."""
    import torch

    rows, k, V = base_logits.shape
    R = w1.shape[1]
    sh = make_shape(rows, V, R, mult, softcap)
    args = (
        _dev(base_logits, torch.bfloat16, "base_logits"),
        _dev(w1, torch.bfloat16, "w1", (V, R)),
        _dev(w2, torch.bfloat16, "w2", (V, R)),
        _dev(prev, torch.int64, "prev", (rows,)),
        _dev(seeds, torch.int64, "seeds", (rows,)),
        _dev(positions, torch.int64, "positions", (rows, k)),
        ctypes.c_int32(k),
        _dev(temperature, torch.float32, "temperature", (rows,)),
        _dev(cache, torch.bfloat16, "cache", (rows, k, V)),
        _dev(tokens, torch.int64, "tokens", (rows, k)),
        _stream_ptr(stream),
        ctypes.byref(sh),
        _dev(workspace, torch.uint8, "workspace"),
        ctypes.c_size_t(workspace.numel()),
    )
    if step is not None:
        args = args[:7] + (ctypes.c_int32(step),) + args[7:]
        _check(lib().markov_sample_step(*args), "markov_sample_step")
        return
    fn = (lib().markov_debug_sample_exact if exact else
          lib().markov_debug_sample_fallback if fallback else lib().markov_sample_sequential)
    _check(fn(*args), "markov_sample_sequential")


def sample_sequential_noalloc(base_logits, w1, w2, prev, seeds, positions, temperature, cache,
                              tokens, mult: float = 1.0, softcap: float = 0.0, stream=None):
    """markov_sample_sequential_noalloc: the loop with the library's own
    per-device workspace (no workspace argument, nothing allocated)."""
    import torch

    rows, k, V = base_logits.shape
    R = w1.shape[1]
    sh = make_shape(rows, V, R, mult, softcap)
    _check(lib().markov_sample_sequential_noalloc(
        _dev(base_logits, torch.bfloat16, "base_logits"),
        _dev(w1, torch.bfloat16, "w1", (V, R)),
        _dev(w2, torch.bfloat16, "w2", (V, R)),
        _dev(prev, torch.int64, "prev", (rows,)),
        _dev(seeds, torch.int64, "seeds", (rows,)),
        _dev(positions, torch.int64, "positions", (rows, k)),
        ctypes.c_int32(k),
        _dev(temperature, torch.float32, "temperature", (rows,)),
        _dev(cache, torch.bfloat16, "cache", (rows, k, V)),
        _dev(tokens, torch.int64, "tokens", (rows, k)),
        _stream_ptr(stream), ctypes.byref(sh)), "markov_sample_sequential_noalloc")


def _opt(t, dtype, name, shape=None):
    return ctypes.c_void_p(None) if t is None else _dev(t, dtype, name, shape)


def greedy_sequential(base_logits, w1, w2, prev, tokens, workspace, cache=None, winners=None,
                      mult: float = 1.0, softcap: float = 0.0, stream=None,
                      step: int | None = None):
    """markov_greedy_sequential: every row at temperature 0. base_logits bf16
    [rows, k, V]; cache bf16 [rows, k, V] or None (not written); tokens int64
    [rows, k]; winners int64 [rows, k] (the packed u64 winners, as int64
    bits) or None; ``step`` runs that one step alone (markov_greedy_step)."""
    import torch

    rows, k, V = base_logits.shape
    R = w1.shape[1]
    sh = make_shape(rows, V, R, mult, softcap)
    head = (_dev(base_logits, torch.bfloat16, "base_logits"), _dev(w1, torch.bfloat16, "w1", (V, R)),
            _dev(w2, torch.bfloat16, "w2", (V, R)), _dev(prev, torch.int64, "prev", (rows,)),
            ctypes.c_int32(k))
    tail = (_opt(cache, torch.bfloat16, "cache", (rows, k, V)),
            _dev(tokens, torch.int64, "tokens", (rows, k)),
            _opt(winners, torch.int64, "winners", (rows, k)),
            _stream_ptr(stream), ctypes.byref(sh), _dev(workspace, torch.uint8, "workspace"),
            ctypes.c_size_t(workspace.numel()))
    if step is not None:
        _check(lib().markov_greedy_step(*head, ctypes.c_int32(step), *tail), "markov_greedy_step")
    else:
        _check(lib().markov_greedy_sequential(*head, *tail), "markov_greedy_sequential")


def greedy_finalize(winners, tokens, stream=None):
    """markov_greedy_finalize: token ids of packed winners (int64 tensors of
    the same number of elements)."""
    import torch

    if winners.numel() != tokens.numel():
        raise ValueError("greedy_finalize: winners and tokens differ in size")
    _check(lib().markov_greedy_finalize(_dev(winners, torch.int64, "winners"), winners.numel(),
                                        _dev(tokens, torch.int64, "tokens"), _stream_ptr(stream)),
           "markov_greedy_finalize")


def quantize_w2_fp8(w2, w2q, w2_scales, stream=None):
    """markov_quantize_w2_fp8: w2 bf16 [V, R] -> w2q uint8 [V, R], w2_scales
    int16 [V] (FP16 bit patterns)."""
    import torch

    V, R = w2.shape
    _check(lib().markov_quantize_w2_fp8(_dev(w2, torch.bfloat16, "w2"),
                                        _dev(w2q, torch.uint8, "w2q", (V, R)),
                                        _dev(w2_scales, torch.int16, "w2_scales", (V,)), V, R,
                                        _stream_ptr(stream)), "markov_quantize_w2_fp8")


def sample_sequential_fp8(base_logits, w1, w2q, w2_scales, prev, seeds, positions, temperature,
                          cache, tokens, workspace, mult: float = 1.0, softcap: float = 0.0,
                          stream=None):
    """markov_sample_sequential_fp8 (arguments as sample_sequential, with the
    E4M3 w2 of ``quantize_w2_fp8`` for w2)."""
    import torch

    rows, k, V = base_logits.shape
    R = w1.shape[1]
    sh = make_shape(rows, V, R, mult, softcap)
    _check(lib().markov_sample_sequential_fp8(
        _dev(base_logits, torch.bfloat16, "base_logits"), _dev(w1, torch.bfloat16, "w1", (V, R)),
        _dev(w2q, torch.uint8, "w2q", (V, R)), _dev(w2_scales, torch.int16, "w2_scales", (V,)),
        _dev(prev, torch.int64, "prev", (rows,)), _dev(seeds, torch.int64, "seeds", (rows,)),
        _dev(positions, torch.int64, "positions", (rows, k)), ctypes.c_int32(k),
        _dev(temperature, torch.float32, "temperature", (rows,)),
        _dev(cache, torch.bfloat16, "cache", (rows, k, V)),
        _dev(tokens, torch.int64, "tokens", (rows, k)), _stream_ptr(stream), ctypes.byref(sh),
        _dev(workspace, torch.uint8, "workspace"), ctypes.c_size_t(workspace.numel())),
        "markov_sample_sequential_fp8")


def greedy_sequential_fp8(base_logits, w1, w2q, w2_scales, prev, tokens, workspace, cache=None,
                          winners=None, mult: float = 1.0, softcap: float = 0.0, stream=None):
    """markov_greedy_sequential_fp8 (as greedy_sequential, E4M3 w2)."""
    import torch

    rows, k, V = base_logits.shape
    R = w1.shape[1]
    sh = make_shape(rows, V, R, mult, softcap)
    _check(lib().markov_greedy_sequential_fp8(
        _dev(base_logits, torch.bfloat16, "base_logits"), _dev(w1, torch.bfloat16, "w1", (V, R)),
        _dev(w2q, torch.uint8, "w2q", (V, R)), _dev(w2_scales, torch.int16, "w2_scales", (V,)),
        _dev(prev, torch.int64, "prev", (rows,)), ctypes.c_int32(k),
        _opt(cache, torch.bfloat16, "cache", (rows, k, V)),
        _dev(tokens, torch.int64, "tokens", (rows, k)),
        _opt(winners, torch.int64, "winners", (rows, k)), _stream_ptr(stream), ctypes.byref(sh),
        _dev(workspace, torch.uint8, "workspace"), ctypes.c_size_t(workspace.numel())),
        "markov_greedy_sequential_fp8")


def debug_e4m3_encode(x, out, stream=None):
    import torch

    _check(lib().markov_debug_e4m3_encode(_dev(x, torch.float32, "x"), _dev(out, torch.uint8, "out"),
                                          x.numel(), _stream_ptr(stream)), "markov_debug_e4m3_encode")


def debug_e4m3_decode(codes, out, stream=None):
    import torch

    _check(lib().markov_debug_e4m3_decode(_dev(codes, torch.uint8, "codes"),
                                          _dev(out, torch.int16, "out"), codes.numel(),
                                          _stream_ptr(stream)), "markov_debug_e4m3_decode")


def debug_bias_fp8(w1, w2q, w2_scales, tok, bias, stream=None):
    import torch

    V, R = w1.shape
    rows = tok.shape[0]
    sh = make_shape(rows, V, R)
    _check(lib().markov_debug_bias_fp8(_dev(w1, torch.bfloat16, "w1"), _dev(w2q, torch.uint8, "w2q"),
                                       _dev(w2_scales, torch.int16, "w2_scales"),
                                       _dev(tok, torch.int64, "tok"),
                                       _dev(bias, torch.bfloat16, "bias", (rows, V)),
                                       ctypes.byref(sh), _stream_ptr(stream)), "markov_debug_bias_fp8")


def shard_step(base_logits, w1, w2, feed, seeds, positions, temperature, cache, packets,
               workspace, step: int, vocab_offset: int, feed_stride: int = 1, mult: float = 1.0,
               softcap: float = 0.0, stream=None):
    """markov_shard_step: base_logits / cache bf16 [rows, k, Vs] (this slab),
    w1 bf16 [V_total, R], w2 bf16 [Vs, R] (this slab), feed int64 (row r at
    feed[r * feed_stride]), packets int64 [rows] (u64 bits)."""
    import torch

    rows, k, Vs = base_logits.shape
    Vt, R = w1.shape
    sh = make_shape(rows, Vs, R, mult, softcap)
    _check(lib().markov_shard_step(
        _dev(base_logits, torch.bfloat16, "base_logits"), _dev(w1, torch.bfloat16, "w1"),
        _dev(w2, torch.bfloat16, "w2", (Vs, R)), _dev(feed, torch.int64, "feed"),
        int(feed_stride), _dev(seeds, torch.int64, "seeds", (rows,)),
        _dev(positions, torch.int64, "positions", (rows, k)), ctypes.c_int32(k),
        ctypes.c_int32(step), _dev(temperature, torch.float32, "temperature", (rows,)),
        _dev(cache, torch.bfloat16, "cache", (rows, k, Vs)),
        _dev(packets, torch.int64, "packets", (rows,)), ctypes.c_int32(vocab_offset),
        ctypes.c_int32(Vt), _stream_ptr(stream), ctypes.byref(sh),
        _dev(workspace, torch.uint8, "workspace"), ctypes.c_size_t(workspace.numel())),
        "markov_shard_step")


def pick(packets, tokens, stride: int = 1, winner=None, stream=None):
    """markov_pick: packets int64 [G, rows] (u64 bits); tokens int64 (row r's
    global token at tokens[r * stride])."""
    import torch

    G, rows = packets.shape
    _check(lib().markov_pick(_dev(packets, torch.int64, "packets"), G, rows,
                             _dev(tokens, torch.int64, "tokens"), int(stride),
                             _opt(winner, torch.int64, "winner", (rows,)), _stream_ptr(stream)),
           "markov_pick")


def new_verify_workspace(batch: int, proposal_len: int, device="cuda"):
    """A zeroed workspace for the verifiers (uint8 tensor)."""
    import torch

    n = int(lib().markov_verify_workspace_bytes(int(batch), int(proposal_len)))
    if n == 0:
        raise MarkovError(-2, "markov_verify_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def greedy_accept(target_logits, draft, proposal_lengths, accepted, accept_len, workspace,
                  stream=None):
    """markov_greedy_accept: target_logits bf16 [B, P+1, V]; draft int64 [B, S]
    (S >= P); proposal_lengths int32 [B]; accepted int64 [B, P+1]; accept_len
    int32 [B]."""
    import torch

    B, P1, V = target_logits.shape
    _check(lib().markov_greedy_accept(
        _dev(target_logits, torch.bfloat16, "target_logits"), _dev(draft, torch.int64, "draft"),
        draft.shape[1], _dev(proposal_lengths, torch.int32, "proposal_lengths", (B,)),
        _dev(accepted, torch.int64, "accepted", (B, P1)),
        _dev(accept_len, torch.int32, "accept_len", (B,)), B, P1 - 1, V,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream_ptr(stream)),
        "markov_greedy_accept")


def prob_accept(target_probs, draft_probs, draft, proposal_lengths, uniforms, accepted,
                accept_len, workspace, stream=None):
    """markov_prob_accept: target_probs fp32 [B, P+1, V]; draft_probs fp32
    [B, P, V]; draft int64 [B, S]; proposal_lengths int32 [B]; uniforms fp32
    [B, 2P+1]; accepted int64 [B, P+1]; accept_len int32 [B]."""
    import torch

    B, P1, V = target_probs.shape
    P = P1 - 1
    _check(lib().markov_prob_accept(
        _dev(target_probs, torch.float32, "target_probs"),
        _dev(draft_probs, torch.float32, "draft_probs", (B, P, V)), _dev(draft, torch.int64, "draft"),
        draft.shape[1], _dev(proposal_lengths, torch.int32, "proposal_lengths", (B,)),
        _dev(uniforms, torch.float32, "uniforms", (B, 2 * P + 1)),
        _dev(accepted, torch.int64, "accepted", (B, P1)),
        _dev(accept_len, torch.int32, "accept_len", (B,)), B, P, V,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream_ptr(stream)),
        "markov_prob_accept")


def noalloc_max_rows() -> int:
    return int(lib().markov_noalloc_max_rows())


def debug_bias(w1, w2, tok, bias, stream=None):
    import torch

    V, R = w1.shape
    rows = tok.shape[0]
    sh = make_shape(rows, V, R)
    _check(lib().markov_debug_bias(_dev(w1, torch.bfloat16, "w1"), _dev(w2, torch.bfloat16, "w2"),
                                   _dev(tok, torch.int64, "tok"),
                                   _dev(bias, torch.bfloat16, "bias", (rows, V)),
                                   ctypes.byref(sh), _stream_ptr(stream)), "markov_debug_bias")


def debug_gumbel(logits, ids, temperature: float, seed: int, step: int, position: int,
                 workspace, key_exact, key_upper, stream=None):
    """Exact keys and the kernel's upper bounds of (logit, id) pairs of one
    row at one step; `workspace` from ``new_workspace``."""
    import torch

    n = logits.numel()
    _check(lib().markov_debug_gumbel(
        _dev(logits, torch.float32, "logits"), _dev(ids, torch.int32, "ids"), n,
        float(temperature), int(seed), int(step), int(position),
        _dev(workspace, torch.uint8, "workspace"),
        _dev(key_exact, torch.float32, "key_exact"), _dev(key_upper, torch.float32, "key_upper"),
        _stream_ptr(stream)), "markov_debug_gumbel")


def debug_bf16_round(x, out, stream=None):
    import torch

    _check(lib().markov_debug_bf16_round(_dev(x, torch.float32, "x"), _dev(out, torch.int16, "out"),
                                         x.numel(), _stream_ptr(stream)),
           "markov_debug_bf16_round")


# The workspace starts with the noise bound tables: 2176 (A, B) float32
# pairs (the per-bucket lines), then 2112 float32 constants (each bucket's
# largest noise plus 1e-5); then the output-transform table (a 256-byte
# stamp, 32768 bf16 entries); then a 256-byte block with the last step's
# completion count and the per-row slot arrays, both zero between calls
# (TABLES_BYTES is where that zero part starts).
TABLE_PAIRS_BYTES = 2176 * 8
NOISE_TABLES_BYTES = TABLE_PAIRS_BYTES + 2112 * 4
TRANSFORM_STAMP_BYTES = 256
TRANSFORM_ENTRIES = 32768
TABLES_BYTES = NOISE_TABLES_BYTES + TRANSFORM_STAMP_BYTES + 2 * TRANSFORM_ENTRIES


def debug_transform_table(mult: float, softcap: float):
    """The output-transform table the library builds for (mult, softcap) as a
    host numpy uint16 array [32768] (bf16 bits; entry i for the sum of bits i)."""
    import numpy as np

    out = np.zeros(TRANSFORM_ENTRIES, dtype=np.uint16)
    n = lib().markov_debug_transform_table(ctypes.c_float(mult), ctypes.c_float(softcap),
                                           out.ctypes.data_as(ctypes.c_void_p), TRANSFORM_ENTRIES)
    if n != TRANSFORM_ENTRIES:
        raise MarkovError(int(n) if n < 0 else -2, "markov_debug_transform_table")
    return out


def debug_noise_table():
    """The noise bound tables as a host numpy float32 array [2050, 3]: per
    bucket the line's A and B (bound = fma(B, float(h), A)) and the constant
    bound C."""
    import numpy as np

    out = np.zeros((2050, 3), dtype=np.float32)
    n = lib().markov_debug_noise_table(out.ctypes.data_as(ctypes.c_void_p), 2050)
    if n != 2050:
        raise MarkovError(int(n) if n < 0 else -2, "markov_debug_noise_table")
    return out


def debug_copy(src, dst, stream=None):
    """A plain device copy of src into dst (same byte size; counter calibration)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("debug_copy: src and dst differ in size")
    _check(lib().markov_debug_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                   n, _stream_ptr(stream)), "markov_debug_copy")


class PreparedCall:
    """A loop (or one step) with its arguments marshalled once, for tight
    launch loops and graph capture. Calling it enqueues the kernels on the
    stream it was prepared for."""

    def __init__(self, fn, args, stream_index, what):
        self._fn, self._args, self._si, self._what = fn, list(args), stream_index, what

    def on(self, stream):
        c = PreparedCall(self._fn, self._args, self._si, self._what)
        c._args[self._si] = _stream_ptr(stream)
        return c

    def __call__(self):
        _check(self._fn(*self._args), self._what)


def prepare_greedy(w, d, cache: bool = True, winners=None, stream=None,
                   step: int | None = None) -> PreparedCall:
    """Marshal a greedy loop (or one step) of workload `w` on device tensors
    `d` once; ``cache`` False leaves the cache unwritten."""
    import torch

    rows, k, V, R = w.rows, w.k, w.V, w.R
    sh = make_shape(rows, V, R, w.mult, w.softcap)
    args = [
        _dev(d["base"], torch.bfloat16, "base_logits", (rows, k, V)),
        _dev(d["w1"], torch.bfloat16, "w1", (V, R)),
        _dev(d["w2"], torch.bfloat16, "w2", (V, R)),
        _dev(d["prev"], torch.int64, "prev", (rows,)),
        ctypes.c_int32(k),
        _dev(d["cache"], torch.bfloat16, "cache", (rows, k, V)) if cache else ctypes.c_void_p(None),
        _dev(d["tokens"], torch.int64, "tokens", (rows, k)),
        _opt(winners, torch.int64, "winners", (rows, k)),
        _stream_ptr(stream),
        ctypes.byref(sh),
        _dev(d["workspace"], torch.uint8, "workspace"),
        ctypes.c_size_t(d["workspace"].numel()),
    ]
    if step is not None:
        args.insert(5, ctypes.c_int32(step))
        call = PreparedCall(lib().markov_greedy_step, args, 9, "markov_greedy_step")
    else:
        call = PreparedCall(lib().markov_greedy_sequential, args, 8, "markov_greedy_sequential")
    call._keep = sh
    return call


def prepare_fp8(w, d, greedy: bool = False, stream=None, step: int | None = None) -> PreparedCall:
    """Marshal an E4M3-w2 loop (or one step) of workload `w` on device tensors
    `d` (with d["w2q"], d["w2s"] from quantize_w2_fp8) once."""
    import torch

    rows, k, V, R = w.rows, w.k, w.V, w.R
    sh = make_shape(rows, V, R, w.mult, w.softcap)
    head = [
        _dev(d["base"], torch.bfloat16, "base_logits", (rows, k, V)),
        _dev(d["w1"], torch.bfloat16, "w1", (V, R)),
        _dev(d["w2q"], torch.uint8, "w2q", (V, R)),
        _dev(d["w2s"], torch.int16, "w2_scales", (V,)),
        _dev(d["prev"], torch.int64, "prev", (rows,)),
    ]
    tail = [_stream_ptr(stream), ctypes.byref(sh), _dev(d["workspace"], torch.uint8, "workspace"),
            ctypes.c_size_t(d["workspace"].numel())]
    st = [ctypes.c_int32(step)] if step is not None else []
    if greedy:
        args = head + [ctypes.c_int32(k)] + st + [
            _dev(d["cache"], torch.bfloat16, "cache", (rows, k, V)),
            _dev(d["tokens"], torch.int64, "tokens", (rows, k)), ctypes.c_void_p(None)] + tail
        fn = lib().markov_greedy_step_fp8 if step is not None else lib().markov_greedy_sequential_fp8
    else:
        args = head + [_dev(d["seeds"], torch.int64, "seeds", (rows,)),
                       _dev(d["positions"], torch.int64, "positions", (rows, k)),
                       ctypes.c_int32(k)] + st + [
            _dev(d["temperature"], torch.float32, "temperature", (rows,)),
            _dev(d["cache"], torch.bfloat16, "cache", (rows, k, V)),
            _dev(d["tokens"], torch.int64, "tokens", (rows, k))] + tail
        fn = lib().markov_sample_step_fp8 if step is not None else lib().markov_sample_sequential_fp8
    call = PreparedCall(fn, args, len(args) - 4, "fp8 loop")
    call._keep = sh
    return call


def prepare(w, d, step: int | None = None, exact: bool = False, stream=None,
            fallback: bool = False) -> PreparedCall:
    """Marshal the arguments of workload `w` on device tensors `d` (see
    ``workloads.to_device``) once."""
    import torch

    rows, k, V, R = w.rows, w.k, w.V, w.R
    sh = make_shape(rows, V, R, w.mult, w.softcap)
    args = [
        _dev(d["base"], torch.bfloat16, "base_logits", (rows, k, V)),
        _dev(d["w1"], torch.bfloat16, "w1", (V, R)),
        _dev(d["w2"], torch.bfloat16, "w2", (V, R)),
        _dev(d["prev"], torch.int64, "prev", (rows,)),
        _dev(d["seeds"], torch.int64, "seeds", (rows,)),
        _dev(d["positions"], torch.int64, "positions", (rows, k)),
        ctypes.c_int32(k),
        _dev(d["temperature"], torch.float32, "temperature", (rows,)),
        _dev(d["cache"], torch.bfloat16, "cache", (rows, k, V)),
        _dev(d["tokens"], torch.int64, "tokens", (rows, k)),
        _stream_ptr(stream),
        sh,
        _dev(d["workspace"], torch.uint8, "workspace"),
        ctypes.c_size_t(d["workspace"].numel()),
    ]
    args[11] = ctypes.byref(sh)
    keep = sh
    si = 10
    if step is not None:
        args.insert(7, ctypes.c_int32(step))
        si = 11
        call = PreparedCall(lib().markov_sample_step, args, si, "markov_sample_step")
    else:
        fn = (lib().markov_debug_sample_exact if exact else
              lib().markov_debug_sample_fallback if fallback else lib().markov_sample_sequential)
        call = PreparedCall(fn, args, si, "markov_sample_sequential")
    call._keep = keep
    return call
