"""The binding checks, before anything reaches the library, that every device
tensor covers the extent the call will touch for the sizes it passes and that
it sits on the current device (the library receives raw pointers and sizes
only). Runs without a GPU: tensors are stand-ins that report a shape, an
element size and a device, and the library is replaced by a guard that
fails the test if any entry point is reached with a bad argument."""

import types

import numpy as np
import pytest

from bit_quantized_linear_amd import binding as b

M, K, N, R = 40, 128, 64, 16
G = K // 64


class Dev:
    """Stand-in for a contiguous torch tensor on a GPU."""

    def __init__(self, shape, itemsize, device=0):
        self.shape = tuple(shape)
        self._itemsize = itemsize
        self.device = types.SimpleNamespace(index=device)
        self.is_cuda = True

    def dim(self):
        return len(self.shape)

    def numel(self):
        return int(np.prod(self.shape))

    def element_size(self):
        return self._itemsize

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 0x10000


class Reached(Exception):
    pass


class GuardLib:
    """Size queries go to the real library; an entry point raises Reached."""

    SIZE = {"svdq_qrow_bytes", "svdq_mx_scale_ld", "w4a16_weight_bytes", "svdq_act_workspace_bytes",
            "svdq_mlp_workspace_bytes", "w8a8_workspace_bytes", "svdq_status_string"}

    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name in self.SIZE:
            return getattr(self.real, name)

        def entry(*args):
            raise Reached(name)

        return entry


@pytest.fixture
def guarded(monkeypatch):
    real = b.lib()
    guard = GuardLib(real)
    monkeypatch.setattr(b, "lib", lambda: guard)
    monkeypatch.setattr(b, "_current_device", lambda: 0)
    monkeypatch.setattr(b, "_stream", lambda s: None)
    return guard


def _calls():
    """name -> (function, {argument: tensor}, extra positional args builder)."""
    R6 = b.lib().svdq_qrow_bytes(K, b.QFMT_FP6)
    R6n = b.lib().svdq_qrow_bytes(N, b.QFMT_FP6)
    ldm, ldn = b.lib().svdq_mx_scale_ld(M), b.lib().svdq_mx_scale_ld(N)
    w16 = b.lib().w4a16_weight_bytes(K, N)
    mlp_ws = b.lib().svdq_mlp_workspace_bytes(M, N, R)
    w8_ws = b.lib().w8a8_workspace_bytes(M, K)
    return {
        "channel_absmax": (lambda t: b.svdq_channel_absmax(t["X"], t["absmax"]),
                           {"X": Dev((M, K), 2), "absmax": Dev((K,), 4)}),
        "quantize_act": (lambda t: b.svdq_quantize_act(t["X"], t["smooth"], t["l1t"], t["qx"], t["sx"], t["T"], R,
                                                       qfmt=b.QFMT_FP6),
                         {"X": Dev((M, K), 2), "smooth": Dev((K,), 4), "l1t": Dev((R, K), 2),
                          "qx": Dev((M, R6), 1), "sx": Dev((G, M), 4), "T": Dev((M, R), 2)}),
        "quantize_act_noalloc": (lambda t: b.svdq_quantize_act_noalloc(t["X"], t["smooth"], t["l1t"], t["qx"], t["sx"],
                                                                       t["T"], R, qfmt=b.QFMT_FP6),
                                 {"X": Dev((M, K), 2), "smooth": Dev((K,), 4), "l1t": Dev((R, K), 2),
                                  "qx": Dev((M, R6), 1), "sx": Dev((G, M), 4), "T": Dev((M, R), 2)}),
        "w4a4_linear": (lambda t: b.svdq_w4a4_linear(t["qx"], t["sx"], t["T"], t["qw"], t["sw"], t["l2t"], t["bias"],
                                                     t["Y"], M, N, K, R, qfmt=b.QFMT_FP6),
                        {"qx": Dev((M, R6), 1), "sx": Dev((G, M), 4), "T": Dev((M, R), 2), "qw": Dev((N, R6), 1),
                         "sw": Dev((G, N), 4), "l2t": Dev((N, R), 2), "bias": Dev((N,), 2), "Y": Dev((M, N), 4)}),
        "gelu_quantize": (lambda t: b.svdq_w4a4_linear_gelu_quantize(
            t["qx"], t["sx"], t["T"], t["qw"], t["sw"], t["l2t"], t["bias"], M, N, K, R, t["smooth_down"],
            t["l1t_down"], R, t["qx_down"], t["sx_down"], t["T_down"], t["Y_up"], t["workspace"]),
            {"qx": Dev((M, R6), 1), "sx": Dev((G, M), 4), "T": Dev((M, R), 2), "qw": Dev((N, R6), 1),
             "sw": Dev((G, N), 4), "l2t": Dev((N, R), 2), "bias": Dev((N,), 2), "smooth_down": Dev((N,), 4),
             "l1t_down": Dev((R, N), 2), "qx_down": Dev((M, R6n), 1), "sx_down": Dev((N // 64, M), 4),
             "T_down": Dev((M, R), 2), "Y_up": Dev((M, N), 2), "workspace": Dev((mlp_ws,), 1)}),
        "w8a8_linear": (lambda t: b.w8a8_linear(t["X"], t["qw"], 0.5, t["bias"], t["workspace"], t["Y"]),
                        {"X": Dev((M, K), 2), "qw": Dev((N, K), 1), "bias": Dev((N,), 2),
                         "workspace": Dev((w8_ws,), 1), "Y": Dev((M, N), 2)}),
        "mx_quantize_act": (lambda t: b.svdq_mx_quantize_act(t["X"], t["smooth"], t["l1t"], t["qx"], t["ux"], t["T"], R),
                            {"X": Dev((M, K), 2), "smooth": Dev((K,), 4), "l1t": Dev((R, K), 2),
                             "qx": Dev((M, K // 2), 1), "ux": Dev((K // 32, ldm), 1), "T": Dev((M, R), 2)}),
        "mx_linear": (lambda t: b.svdq_mx_linear(t["qx"], t["ux"], t["T"], t["qw"], t["uw"], t["l2t"], t["bias"],
                                                 t["Y"], M, N, K, R),
                      {"qx": Dev((M, K // 2), 1), "ux": Dev((K // 32, ldm), 1), "T": Dev((M, R), 2),
                       "qw": Dev((N, K // 2), 1), "uw": Dev((K // 32, ldn), 1), "l2t": Dev((N, R), 2),
                       "bias": Dev((N,), 2), "Y": Dev((M, N), 2)}),
        "w4a16_linear": (lambda t: b.w4a16_linear(t["X"], t["packed"], t["bias"], t["Y"], N),
                         {"X": Dev((2, K), 2), "packed": Dev((w16,), 1), "bias": Dev((N,), 2), "Y": Dev((2, N), 2)}),
        "group_partials": (lambda t: b.svdq_debug_group_partials(t["qx"], t["qw"], t["P"], M, N, K, qfmt=b.QFMT_FP6),
                           {"qx": Dev((M, R6), 1), "qw": Dev((N, R6), 1), "P": Dev((G, M, N), 4)}),
        "w8a8_acc": (lambda t: b.w8a8_debug_acc(t["qx"], t["qw"], t["acc"], M, N, K),
                     {"qx": Dev((M, K), 1), "qw": Dev((N, K), 1), "acc": Dev((M, N), 4)}),
        "gelu": (lambda t: b.svdq_debug_gelu_bf16(t["y"], t["g"]), {"y": Dev((100,), 2), "g": Dev((100,), 2)}),
    }


CALLS = ["channel_absmax", "gelu", "gelu_quantize", "group_partials", "mx_linear", "mx_quantize_act",
         "quantize_act", "quantize_act_noalloc", "w4a16_linear", "w4a4_linear", "w8a8_acc", "w8a8_linear"]


def test_the_call_list_is_complete():
    assert sorted(_calls()) == CALLS


@pytest.mark.parametrize("call", CALLS)
def test_well_sized_arguments_reach_the_library(call, guarded):
    fn, tensors = _calls()[call]
    with pytest.raises(Reached):
        fn(tensors)


def _shrunk(t):
    """The same tensor one element short (its last dimension cut by one)."""
    return Dev(t.shape[:-1] + (t.shape[-1] - 1,), t.element_size(), t.device.index)


@pytest.mark.parametrize("call", CALLS)
def test_an_undersized_tensor_is_refused_before_any_launch(call, guarded):
    fn, tensors = _calls()[call]
    # the input whose shape defines the call's sizes cannot be undersized
    defining = {"X", "y"}
    for name in tensors:
        if name in defining:
            continue
        bad = dict(tensors)
        bad[name] = _shrunk(tensors[name])
        with pytest.raises(ValueError, match=name):
            fn(bad)


@pytest.mark.parametrize("call", CALLS)
def test_a_tensor_on_another_device_is_refused(call, guarded):
    fn, tensors = _calls()[call]
    for name, t in tensors.items():
        bad = dict(tensors)
        bad[name] = Dev(t.shape, t.element_size(), device=1)
        with pytest.raises(TypeError, match="current device"):
            fn(bad)


def test_wrong_element_size_is_refused(guarded):
    fn, tensors = _calls()["w4a4_linear"]
    bad = dict(tensors)
    bad["sx"] = Dev((G * 2, M), 2)  # same bytes, 2-byte elements
    with pytest.raises(TypeError, match="4-byte"):
        fn(bad)
