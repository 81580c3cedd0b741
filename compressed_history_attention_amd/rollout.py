"""Multi-layer rollout driver over libnanokv's per-layer cache calls.

An autoregressive video rollout produces one chunk at a time.  While a chunk
is generated, every attention layer reads that layer's compressed history
together with the chunk's own keys/values (NanoKV: High-Ratio KV Cache
Compression for Autoregressive Video Generation, Figure 4(a) and (d)); when
the chunk is final its K and V are encoded and appended to every layer's
history (Figure 4(b)).  Each layer has its own full-dimensional routing
policy (Table 7: recent frames, anchors, sinks, full-layer fallback) and its
own per-head low-dimensional widths (Table 6).

The driver owns the per-layer caches (torch device memory) and loops over
layers; every step runs in the library's kernels (``nkv_layer_attend`` and
``nkv_layer_append``).  There is no backbone here: the caller supplies each
layer's queries, keys and values.
"""
from __future__ import annotations

from typing import List, Sequence

import torch

from . import lib
from .lib import LayerCache, RoutePolicy, Shape


class Rollout:
    """Compressed histories of ``len(codecs)`` layers.

    codecs[l] = (centers (K, V), encoders (K, V), decoders (K, V)) as device
    tensors of the shape's dtype; policies[l] a RoutePolicy; widths[l] one
    low-dimensional width for every head or a list of H widths.
    """

    def __init__(self, shape: Shape, codecs, policies: Sequence[RoutePolicy], widths,
                 capacity: int, device="cuda"):
        if len(codecs) != len(policies) or len(codecs) != len(widths):
            raise ValueError("need one codec, policy and width setting per layer")
        self.shape = shape
        self.policies = list(policies)
        self.widths = [self._per_head(w) for w in widths]
        self.caches: List[LayerCache] = [
            LayerCache(shape, capacity, c[0], c[1], c[2], device) for c in codecs]
        self.device = torch.device(device)
        self._ws = torch.empty(0, dtype=torch.uint8, device=self.device)

    def _per_head(self, w):
        if isinstance(w, int):
            return [w] * self.shape.H
        w = [int(x) for x in w]
        if len(w) != self.shape.H:
            raise ValueError(f"need {self.shape.H} widths per layer")
        return w

    @property
    def layers(self) -> int:
        return len(self.caches)

    @property
    def n_hist(self) -> int:
        return self.caches[0].n_hist

    def _workspace(self, nbytes: int):
        if nbytes > self._ws.numel():
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws if nbytes else None

    def attend(self, layer: int, q, cur_k, cur_v, out=None, lse=None, stream=None):
        """Attention of one layer for the chunk being generated."""
        sh, c = self.shape, self.caches[layer]
        Nq = int(q.shape[0])
        N_cur = 0 if cur_k is None else int(cur_k.shape[0])
        if out is None:
            out = torch.empty((Nq, sh.W), dtype=sh.torch_dtype, device=q.device)
        if lse is None:
            lse = torch.empty((Nq, sh.H), dtype=torch.float32, device=q.device)
        pol, w = self.policies[layer], self.widths[layer]
        ws = self._workspace(lib.nkv_layer_attend_workspace_size(sh, c, pol, w, Nq, N_cur))
        lib.nkv_layer_attend(sh, c, pol, w, q, cur_k, cur_v, out, lse, ws=ws, stream=stream)
        return out, lse

    def append(self, layer: int, k_new, v_new, stream=None):
        """Encode the finished chunk's K and V into the layer's history."""
        sh, c = self.shape, self.caches[layer]
        ws = self._workspace(lib.nkv_layer_append_workspace_size(sh, c, int(k_new.shape[0])))
        lib.nkv_layer_append(sh, c, k_new, v_new, ws=ws, stream=stream)

    def chunk(self, inputs, stream=None):
        """One chunk: inputs[l] = (q, k, v) of layer l.  Every layer attends
        first (history before this chunk + the chunk itself), then the chunk
        is appended to every layer.  Returns [(O, LSE)] per layer."""
        outs = [self.attend(l, q, k, v, stream=stream) for l, (q, k, v) in enumerate(inputs)]
        for l, (_, k, v) in enumerate(inputs):
            self.append(l, k, v, stream=stream)
        return outs

    def storage(self) -> dict:
        """Persistent bytes over all layers (cached data vs resident
        operators) and the effective compression ratio."""
        tot = None
        for c in self.caches:
            s = lib.nkv_storage_account(self.shape, int(c.codec[0][0].shape[0]),
                                        int(c.codec[0][1].shape[0]), c.n_hist)
            if tot is None:
                tot = {k: v for k, v in s.items() if not k.startswith("cr_")}
                tot["cr_nominal"] = s["cr_nominal"]
            else:
                for k in tot:
                    if not k.startswith("cr_"):
                        tot[k] += s[k]
        tot["cr_effective"] = tot["original"] / tot["total"] if tot["total"] else 0.0
        tot["cr_cached"] = tot["original"] / tot["cached"] if tot["cached"] else 0.0
        return tot
