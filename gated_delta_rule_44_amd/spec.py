"""Speculative decoding through the GDN layer: the control loop around verify, accept and commit.

The loop follows the "mtp/generate.py" page's decode loop: every step runs the last emitted token and
K drafts through gdn_verify_with_checkpoints (the pool is only read), measures the accepted prefix m
with gdn_accept, and commits directly: the checkpoint after token m is copied into the pool
(gdn_state_copy). The fallback the page keeps for a cache without checkpoints replays the accepted
prefix instead, one gdn_decode_step per token; verify checkpoints are bitwise repeated decode steps,
so both end in the same pool bits. A third mode commits without a copy: the checkpoints of a step go
to rows of their own (two sets of rows, used in turn, so that a step reads the rows the previous one
wrote and writes the others), the commit only moves each sequence's row index to its accepted
checkpoint, and finish() copies the current states back into the caller's pool rows. Drafts and the verifier's greedy predictions come from the caller
(the layer has no LM head); token ids pick rows of the caller's table of projected inputs. The bridge
(the "uni_engine.py" page's _bridge) copies the fixed-size recurrent state records from one pool to
another. Every GPU step is a libgdn call; this module only orders them and keeps the counts.
"""
from __future__ import annotations

import time
from dataclasses import dataclass, field

import numpy as np
import torch

from . import GdnDesc, GdnWeights, accept, decode_step, state_copy, state_record_bytes, verify_with_checkpoints


@dataclass(frozen=True)
class BridgeReport:
    seconds: float
    mib: float
    seen_tokens: int


@dataclass(frozen=True)
class VerifyReport:
    generated_tokens: int
    drafted_tokens: int
    accepted_draft_tokens: int
    rejected_blocks: int
    verifier_blocks: int

    @property
    def acceptance_rate(self) -> float:
        return 1.0 if self.drafted_tokens <= 0 else self.accepted_draft_tokens / self.drafted_tokens


def bridge(desc: GdnDesc, dst_state, dst_tail, src_state, src_tail, n: int, seen_tokens: int = 0) -> BridgeReport:
    """Copy n state records (fp32 state and conv tail) from one pool to another, in place; O(1) in context."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    state_copy(desc, dst_state, dst_tail, None, src_state, src_tail, None, n)
    torch.cuda.synchronize()
    return BridgeReport(time.perf_counter() - t0, n * state_record_bytes(desc) / 2 ** 20, int(seen_tokens))


@dataclass
class LoopStats:
    K: int
    B: int = 1
    steps: int = 0
    tokens: int = 0
    drafted: int = 0
    accepted_drafts: int = 0
    rejected_blocks: int = 0
    verifier_blocks: int = 0
    direct_commits: int = 0
    fallback_replays: int = 0
    replayed_tokens: int = 0
    accept_hist: list = field(default_factory=list)  # [sequence steps that matched exactly 0, 1, ..., K drafts]

    def __post_init__(self):
        self.accept_hist = [0] * (self.K + 1)

    def report(self) -> VerifyReport:
        return VerifyReport(self.tokens, self.drafted, self.accepted_drafts, self.rejected_blocks, self.verifier_blocks)

    def as_dict(self) -> dict:
        return {"steps": self.steps, "tokens": self.tokens,
                "avg_accept_len": round(self.tokens / max(self.steps * self.B, 1), 3),
                "direct_commits": self.direct_commits, "fallback_replays": self.fallback_replays,
                "replayed_tokens": self.replayed_tokens, "accept_hist": list(self.accept_hist)}


class SpecDecodeLoop:
    """B sequences in pool rows `slots`, K drafts per step. table: (mixed, z, a, b) projected inputs per
    token id ([V, C_ch], [V, n_v*d_v], [V, n_v], [V, n_v] on the GPU). mode "direct" commits verify
    checkpoints; "replay" decodes the accepted prefix again; "remap" commits by row index (call finish()
    before reading the caller's pool)."""

    def __init__(self, desc: GdnDesc, w: GdnWeights, table, K: int, slots, state_pool, tail_pool, mode="direct"):
        if mode not in ("direct", "replay", "remap"):
            raise ValueError(f"mode {mode!r}")
        self.desc, self.w, self.table, self.K, self.mode = desc, w, table, int(K), mode
        self.state_pool, self.tail_pool = state_pool, tail_pool
        self.slots = torch.as_tensor(np.asarray(slots, np.int32), device=state_pool.device)
        self.B = self.slots.numel()
        T = self.K + 1
        dev = state_pool.device
        self.ck_shape = ((self.B, T, desc.n_v, desc.d_k, desc.d_v), (self.B, T, desc.kc, desc.conv_dim))
        if mode != "remap":
            self.ck_s = torch.empty(self.ck_shape[0], dtype=torch.float32, device=dev)
            self.ck_t = torch.empty(self.ck_shape[1], dtype=desc.act, device=dev)
        self.out = torch.empty(self.B, T, desc.n_v * desc.d_v, dtype=desc.act, device=dev)
        self.stats = LoopStats(self.K, self.B)
        # remap: the rows the sequences' states are in (None: the caller's pool at `slots`), and the two
        # sets of checkpoint rows
        self.cur = None
        self.region = 0
        if mode == "remap":
            self.rows = [(torch.empty(self.B * T, desc.n_v, desc.d_k, desc.d_v, dtype=torch.float32, device=dev),
                          torch.empty(self.B * T, desc.kc, desc.conv_dim, dtype=desc.act, device=dev))
                         for _ in range(2)]

    def _inputs(self, ids: torch.Tensor):
        return [t[ids.long()].contiguous() for t in self.table]

    def step(self, x: np.ndarray, drafts: np.ndarray, preds: np.ndarray):
        """One step. x [B]: the last emitted token of each sequence (not yet in its state); drafts [B,K];
        preds [B,K+1]: the verifier's greedy token after each of the 1+K verify tokens. Returns
        (m [B], emitted [B,K+1] (the first m+1 entries), the verify outputs [B,1+K,n_v*d_v])."""
        B, K, d = self.B, self.K, self.desc
        dev = self.state_pool.device
        ids = torch.as_tensor(np.concatenate([np.asarray(x, np.int32)[:, None], np.asarray(drafts, np.int32)], 1),
                              device=dev)
        mx, zz, aa, bb = self._inputs(ids)
        if self.mode == "remap":
            src_s, src_t, src_idx = self.cur if self.cur is not None else (self.state_pool, self.tail_pool, self.slots)
            dst_s, dst_t = self.rows[self.region]
            verify_with_checkpoints(d, self.w, mx, zz, aa, bb, src_idx, src_t, src_s, dst_s.view(self.ck_shape[0]),
                                    dst_t.view(self.ck_shape[1]), self.out)
        else:
            verify_with_checkpoints(d, self.w, mx, zz, aa, bb, self.slots, self.tail_pool, self.state_pool, self.ck_s,
                                    self.ck_t, self.out)
        dr = torch.as_tensor(np.asarray(drafts, np.int32), device=dev)
        pr = torch.as_tensor(np.asarray(preds, np.int32), device=dev)
        m, em, _, ci = accept(dr, pr)
        m_h, em_h = m.cpu().numpy(), em.cpu().numpy()  # the host needs m to pick the next tokens
        st = self.stats
        if self.mode == "direct":
            state_copy(d, self.state_pool, self.tail_pool, self.slots, self.ck_s, self.ck_t, ci, B)
            st.direct_commits += 1
        elif self.mode == "remap":
            # sequence b's state is now checkpoint row b (1+K) + m_b of this step's rows
            self.cur = (dst_s, dst_t, ci)
            self.region ^= 1
            st.direct_commits += 1
        else:
            # tokens 0 .. m_b of each sequence again, one decode step per position for the sequences that
            # accepted that far
            st.fallback_replays += 1
            for j in range(K + 1):
                sel = np.flatnonzero(m_h >= j)
                if len(sel) == 0:
                    break
                rows = torch.as_tensor(sel, device=dev)
                decode_step(d, self.w, mx[rows, j].contiguous(), zz[rows, j].contiguous(), aa[rows, j].contiguous(),
                            bb[rows, j].contiguous(), self.slots[rows].contiguous(), self.tail_pool, self.state_pool)
                st.replayed_tokens += len(sel)
        st.steps += 1
        st.verifier_blocks += B
        st.drafted += B * K
        st.accepted_drafts += int(m_h.sum())
        st.rejected_blocks += int((m_h < K).sum())
        st.tokens += int((m_h + 1).sum())
        for v in m_h:
            st.accept_hist[int(v)] += 1
        return m_h, em_h, self.out

    def finish(self):
        """remap: copy every sequence's current state into its row of the caller's pool (a no-op otherwise,
        and after the copy the loop reads the caller's pool again)"""
        if self.cur is not None:
            src_s, src_t, src_idx = self.cur
            state_copy(self.desc, self.state_pool, self.tail_pool, self.slots, src_s, src_t, src_idx, self.B)
            self.cur = None
