"""A speculative-decoding round on a stack of MoE layers (the MoE part of MTP
with NEXTN: bpdata.com Ling-3.0-flash MoE article, "Optimalizáció 3": a draft
layer proposes tokens, the target model checks several positions in one
step, and the accepted prefix is kept; the pages run 3 draft steps with 4
draft tokens and report an accept length of 3.90).

The draft and target weights and the acceptance test need trained models, so
the round is emulated with the library's calls only:

  drafts   n_draft steps of the draft layer at M = 1: step d takes row d of
           the verify input (RMS-normalised) and writes its output to row
           d + 1, so each draft builds on the previous one;
  verify   the n_draft + 1 rows through every layer of the stack at once
           (M = n_draft + 1), RMSNorm on each layer's input, as a verify step
           of the target model does.

Which of the drafts would be accepted is left to the caller (the pages'
accept length turns a round time into tokens per second).  This module only
sequences calls of the C ABI through the binding; every step runs in the HIP
kernels, and a round may be captured into a HIP graph.
"""
from __future__ import annotations

from . import binding as B


class MtpRound:
    """Buffers and calls of one round.

    cfg       the layers' MoeConfig
    stack     list of (router_w, packed) of the target's MoE layers
    draft     (router_w, packed) of the draft layer
    ws        a Workspace for at least n_draft + 1 tokens
    """

    def __init__(self, cfg, stack, draft, ws, n_draft: int = 3):
        import torch
        self.cfg, self.stack, self.draft, self.ws, self.n_draft = cfg, list(stack), draft, ws, n_draft
        H, k, M = cfg.hidden, cfg.top_k, n_draft + 1
        dev = "cuda"
        # verify input: row 0 is the round's token input (written by the
        # caller), rows 1.. the draft outputs
        self.rows = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        self.d_ids = torch.empty((1, k), dtype=torch.int32, device=dev)
        self.d_w = torch.empty((1, k), dtype=torch.float32, device=dev)
        self.d_norm = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
        self.v_ids = torch.empty((M, k), dtype=torch.int32, device=dev)
        self.v_w = torch.empty((M, k), dtype=torch.float32, device=dev)
        self.v_norm = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        self.v_bufs = (torch.empty((M, H), dtype=torch.bfloat16, device=dev),
                       torch.empty((M, H), dtype=torch.bfloat16, device=dev))

    @property
    def out(self):
        """The last layer's output of the verify step ([n_draft + 1][H])."""
        return self.v_bufs[(len(self.stack) - 1) % 2]

    def drafts(self, stream=None, record=None):
        """record(d, x_norm, ids, w) is called after each draft step."""
        rt, pk = self.draft
        for d in range(self.n_draft):
            B.layer(self.cfg, rt, pk, self.rows[d:d + 1], self.d_ids, self.d_w, self.rows[d + 1:d + 2], self.ws.buf,
                    flags=B.MOE_F_INPUT_RMSNORM, x_norm=self.d_norm, stream=stream)
            if record is not None:
                record(d, self.d_norm, self.d_ids, self.d_w)

    def verify(self, stream=None, record=None):
        """record(l, x_norm, ids, w, out) is called after each layer (tests
        copy what the chain overwrites)."""
        for l, (rt, pk) in enumerate(self.stack):
            src = self.rows if l == 0 else self.v_bufs[(l - 1) % 2]
            dst = self.v_bufs[l % 2]
            B.layer(self.cfg, rt, pk, src, self.v_ids, self.v_w, dst, self.ws.buf,
                    flags=B.MOE_F_INPUT_RMSNORM, x_norm=self.v_norm, stream=stream)
            if record is not None:
                record(l, self.v_norm, self.v_ids, self.v_w, dst)

    def round(self, stream=None, record_draft=None, record_verify=None):
        self.drafts(stream, record_draft)
        self.verify(stream, record_verify)
