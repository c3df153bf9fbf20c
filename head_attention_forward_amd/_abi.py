"""ctypes signatures of every symbol include/*.h declares (no torch: the
host-sanitizer check loads this file on its own)."""

import ctypes

_P = ctypes.c_void_p
_I = ctypes.c_int
SIG = {
    "sdpa_forward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _I, _P]),
    "mha_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I]),
    "sdpa_decode": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _I, _P,
                         ctypes.c_size_t, _P]),
    "sdpa_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "sdpa_decode_launches": (_I, [_I, _I, _I, _I, _I]),
    "sdpa_decode_timed": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _I, _P,
                               ctypes.c_size_t, _P, _P, _I, _P]),
    "mha_forward": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _I, _P,
                         ctypes.c_size_t, _P]),
    "mha_project_in": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P,
                            ctypes.c_size_t, _P]),
    "mha_attend": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _I, _P, ctypes.c_size_t, _P]),
    "mha_project_out": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, ctypes.c_size_t, _P]),
    "mha_status_str": (ctypes.c_char_p, [_I]),
    "mha_forward_launches": (_I, [_I, _I, _I, _I]),
    "sdpa_forward_timed": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _I,
                                _P, _P, _I, _P]),
    "mha_forward_timed": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _I,
                               _P, ctypes.c_size_t, _P, _P, _I, _P]),
    "add_layernorm_forward": (_I, [_P, _P, _P, _P, _P, _I, _I, ctypes.c_float, _I, _P]),
    "ffn_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "ffn_forward": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, ctypes.c_size_t, _P]),
    "encoder_layer_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "encoder_layer_forward": (_I, [_P] * 14 + [_I] * 7 + [ctypes.c_float, _I, _P, _I, _P,
                                                        ctypes.c_size_t, _P]),
    "encoder_layer_forward_timed": (_I, [_P] * 14 + [_I] * 7 + [ctypes.c_float, _I, _P, _I, _P,
                                                              ctypes.c_size_t, _P, _P, _I, _P]),
    "encoder_layer_launches": (_I, [_I, _I]),
    "embed_positional_forward": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "embed_positional_forward_timed": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P]),
    "sdpa_forward_lse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _I,
                              _P]),
    "sdpa_backward_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "sdpa_backward": (_I, [_P] * 9 + [_I] * 6 + [ctypes.c_float, _I, _P, _I, _P, ctypes.c_size_t, _P]),
    "sdpa_backward_noalloc": (_I, [_P] * 9 + [_I] * 6 + [ctypes.c_float, _I, _P, _I, _P]),
    "sdpa_backward_timed": (_I, [_P] * 9 + [_I] * 6 + [ctypes.c_float, _I, _P, _I, _P,
                                                      ctypes.c_size_t, _P, _P, _I, _P]),
    "mha_train_workspace_bytes": (ctypes.c_size_t, [_I] * 7),
    "mha_forward_train": (_I, [_P] * 7 + [_I] * 8 + [_P, _I, _P, ctypes.c_size_t, _P]),
    "mha_backward_workspace_bytes": (ctypes.c_size_t, [_I] * 9),
    "mha_backward": (_I, [_P] * 13 + [_I] * 8 + [_P, _I, _P, ctypes.c_size_t, _P, ctypes.c_size_t,
                                                 _P]),
    "mha_backward_timed": (_I, [_P] * 13 + [_I] * 8 + [_P, _I, _P, ctypes.c_size_t, _P,
                                                       ctypes.c_size_t, _P, _P, _I, _P]),
    "mha_backward_launches": (_I, [_I]),
    # include/mha_probe.h (measurement aids)
    "mha_floor_probe": (_I, [_I, _P, _P, _P, _P, ctypes.c_size_t, _I, _P]),
    "mha_floor_probe_timed": (_I, [_I, _P, _P, _P, _P, ctypes.c_size_t, _I, _P, _P, _I, _P]),
}

