"""Host-side runtime around the C ABI: device memory for weights and workspace (torch),
the generate loop's schedule, and status checking.  No model arithmetic happens here:
every step of the forward pass, the greedy pick and the token select run in the library.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import torch

from . import abi


class LlamaError(RuntimeError):
    def __init__(self, where: str, status: int):
        super().__init__(f"{where}: {abi.llama_status_str(status)} ({status})")
        self.status = status


def check(where: str, status: int) -> None:
    if status != abi.LLAMA_OK:
        raise LlamaError(where, status)


def make_args(dim, n_layers, n_heads, n_kv_heads, vocab_size, hidden_dim, norm_eps, rope_theta,
              max_batch_size, max_seq_len, dtype: str) -> abi.llama_args:
    return abi.llama_args(dim, n_layers, n_heads, n_kv_heads, vocab_size, hidden_dim,
                          float(norm_eps), float(rope_theta), max_batch_size, max_seq_len,
                          abi.DTYPES[dtype])


def stream_handle(stream: Optional[torch.cuda.Stream] = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class LlamaModel:
    """A ctx over caller-owned device weights (dict layout of synth.gen_weights) and a
    workspace tensor allocated here."""

    def __init__(self, args: abi.llama_args, weights: dict, device="cuda"):
        self.args = args
        self.weights = weights             # keep the borrowed tensors alive
        L = []
        for lw in weights["layers"]:
            L.append(abi.llama_layer_weights(*[lw[n].data_ptr() for n in (
                "attention_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w1", "w2", "w3")]))
        self._layers = (abi.llama_layer_weights * len(L))(*L)
        self._w = abi.llama_weights(weights["tok_embeddings"].data_ptr(), weights["norm"].data_ptr(),
                                    weights["output"].data_ptr(),
                                    ctypes.cast(self._layers, ctypes.POINTER(abi.llama_layer_weights)))
        nbytes = abi.llama_workspace_bytes(args)
        if nbytes == 0:
            check("llama_workspace_bytes", abi.llama_check_args(args))
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        st, ctx = abi.llama_init(args, self._w, self.workspace.data_ptr(), nbytes, stream_handle())
        check("llama_init", st)
        self.ctx = ctx

    def close(self) -> None:
        if self.ctx:
            torch.cuda.synchronize()
            abi.llama_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill(self, tokens: torch.Tensor, bsz: int, seqlen: int, start_pos: int,
                logits: torch.Tensor, all_positions: bool = False, col: int = 0) -> None:
        """tokens: int32 [rows][ld] on the device; reads columns [col, col+seqlen)."""
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        check("llama_prefill", abi.llama_prefill(
            self.ctx, tokens.data_ptr() + 4 * col, tokens.shape[1], bsz, seqlen, start_pos,
            logits.data_ptr(), int(all_positions), stream_handle()))

    def decode_step(self, tokens: torch.Tensor, bsz: int, col: int, start_pos: int,
                    logits: torch.Tensor) -> None:
        """Feeds tokens[:, col] at position start_pos."""
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        check("llama_decode_step", abi.llama_decode_step(
            self.ctx, tokens.data_ptr() + 4 * col, tokens.shape[1], bsz, start_pos,
            logits.data_ptr(), stream_handle()))

    def decode_step_noalloc(self, tokens: torch.Tensor, bsz: int, col: int, start_pos: int,
                            logits: torch.Tensor) -> int:
        """decode_step with the step's scratch in the library's static array (no allocation);
        returns the status code."""
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        return abi.llama_decode_step_noalloc(self.ctx, tokens.data_ptr() + 4 * col, tokens.shape[1], bsz,
                                             start_pos, logits.data_ptr(), stream_handle())


def argmax(logits: torch.Tensor, out: torch.Tensor) -> None:
    bsz, vocab = logits.shape[0], logits.shape[-1]
    check("llama_argmax", abi.llama_argmax(logits.data_ptr(), bsz, vocab, logits.stride(0),
                                           out.data_ptr(), stream_handle()))


def select_next(nxt: torch.Tensor, tokens: torch.Tensor, cur_pos: int, prompt_len: torch.Tensor) -> None:
    check("llama_select_next", abi.llama_select_next(
        nxt.data_ptr(), tokens.data_ptr(), tokens.shape[1], cur_pos, prompt_len.data_ptr(),
        tokens.shape[0], stream_handle()))


def sample_top_p(logits: torch.Tensor, temperature: float, top_p: float, uniform: torch.Tensor,
                 out: torch.Tensor, logprob: torch.Tensor = None) -> None:
    """Temperature + top-p draw per row at the given uniforms (llama_sample_top_p)."""
    check("llama_sample_top_p", abi.llama_sample_top_p(
        logits.data_ptr(), logits.shape[0], logits.shape[1], logits.stride(0), float(temperature),
        float(top_p), uniform.data_ptr(), out.data_ptr(), logprob.data_ptr() if logprob is not None else 0,
        stream_handle()))


class GreedyRun:
    """Device buffers and schedule of one generate call: prompts left-aligned in a pad-filled
    rectangle, one prefill of the shortest prompt, then one single-token call per position;
    prompt tokens are never overwritten.  At temperature 0 the pick is the argmax; above it,
    the temperature + top-p draw with one uniform per (call, row), drawn up front from a
    seeded generator (`uniforms`, on the device) so no step waits on the host."""

    def __init__(self, model: LlamaModel, prompts: Sequence[Sequence[int]], max_gen_len: int,
                 keep_logits: bool = True, pad_id: int = -1, temperature: float = 0.0,
                 top_p: float = 0.9, seed: int = 0):
        self.model = model
        self.bsz = len(prompts)
        self.min_len = min(len(p) for p in prompts)
        max_len = max(len(p) for p in prompts)
        self.total_len = min(model.args.max_seq_len, max_gen_len + max_len)
        tok = torch.full((self.bsz, self.total_len), pad_id, dtype=torch.int32)
        for b, p in enumerate(prompts):
            tok[b, :len(p)] = torch.tensor(p, dtype=torch.int32)
        self.tokens0 = tok.cuda()
        self.tokens = self.tokens0.clone()
        self.prompt_len = torch.tensor([len(p) for p in prompts], dtype=torch.int32).cuda()
        self.n_calls = self.total_len - self.min_len
        V = model.args.vocab_size
        nbuf = self.n_calls if keep_logits else 1
        self.logits = torch.empty((nbuf, self.bsz, V), dtype=torch.float32, device="cuda")
        self.next = torch.empty(self.bsz, dtype=torch.int32, device="cuda")
        self.keep = keep_logits
        self.temperature, self.top_p = float(temperature), float(top_p)
        if self.temperature > 0.0:
            import numpy as np
            u = np.random.Generator(np.random.Philox(seed)).random((self.n_calls, self.bsz), dtype=np.float32)
            self.uniforms = torch.from_numpy(u).cuda()
            self.logprobs = torch.empty((self.n_calls, self.bsz), dtype=torch.float32, device="cuda")

    def reset(self) -> None:
        self.tokens.copy_(self.tokens0)

    def _buf(self, i: int) -> torch.Tensor:
        return self.logits[i if self.keep else 0]

    def _pick(self, i: int, lg: torch.Tensor) -> None:
        if self.temperature > 0.0:
            sample_top_p(lg, self.temperature, self.top_p, self.uniforms[i], self.next, self.logprobs[i])
        else:
            argmax(lg, self.next)

    def prefill(self) -> None:
        lg = self._buf(0)
        self.model.prefill(self.tokens, self.bsz, self.min_len, 0, lg)
        self._pick(0, lg)
        select_next(self.next, self.tokens, self.min_len, self.prompt_len)

    def decode(self, i: int) -> None:
        """Call i >= 1: feeds position cur-1 and fills position cur = min_len + i."""
        cur = self.min_len + i
        lg = self._buf(i)
        self.model.decode_step(self.tokens, self.bsz, cur - 1, cur - 1, lg)
        self._pick(i, lg)
        select_next(self.next, self.tokens, cur, self.prompt_len)

    def run(self) -> None:
        self.prefill()
        for i in range(1, self.n_calls):
            self.decode(i)
