"""Decode-step driver of the SFI path: slow/fast schedule on the host, kernels on two HIP
streams of one GPU.

Step s of every listed sequence is SLOW when s == 0, when its boundary flag is set, or when
`refresh_budget` fast steps have run since its last slow step, and FAST otherwise (es
"Pasos Lentos", zh "2.1 慢快推理框架").  A slow step runs dense attention and then the Selector
and the pack for that layer; a fast step runs two-segment attention over the packed
buffer and the recent window.  With an evidence window of w > 1 queries, a slow step's
dense attention also runs the w - 1 decode queries before the current one (as extra rows
of each KV head's group, so K and V are read once) and the Selector pools their
attention with the current query's.

Overlap (es "3. Optimización del Sistema", zh "2.3 系统级优化"): the
attention of every layer is issued on stream 1; the Selector and pack of layer i are
issued on a Selector stream after an event recorded behind layer i's slow attention, so
they run while stream 1 continues with layer i+1.  There are two Selector streams, used by
alternate layers, so that the short dependent kernels of two layers' Selectors overlap
each other too.  A one-layer stack runs its Selector and pack on stream 1 by default:
nothing could run beside them, and the cross-stream waits would only add latency.  Before layer i's next attention, stream 1 waits for layer i's pack event.
All streams have the default priority.  Before a slow step queues its first Selector-stream
wait, the host lets stream 1 come within one step of it (`paced`), so that no such wait sits in a
queue far ahead of the attention it depends on.

All per-step tables (sequence lengths, recent-window starts, slow/fast row lists) are
built on the host from the seeded flags and copied to the device once, so a step issues
kernels only.

Graphs (`enable_graphs`): every step whose rows are all fast is captured as one HIP graph
holding that step's calls for every layer, with the step's own query, length and
recent-start pointers, so a replay is the kernels alone.  This removes the host cost of
issuing one call per layer, which is larger than a fast call's GPU time.  The first fast
step after a slow step stays call by call (see `step`).

Pack: the packed buffers are either rebuilt at each slow step (sfi_pack) or updated in
place with only the newly selected rows (sfi_pack_update); the engine updates for a stack
of layers and rebuilds for one layer (see `Engine.__init__`).  Step 0 empties them.

Device control (`device_control=True`): the schedule is decided on the device from the
decoded token ids instead (sfi_step_control), the new K/V rows are appended there
(sfi_kv_append), and every step is one graph (`enable_device_graphs`); nothing on the
host depends on the schedule.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import lib as L


def schedule(flags: np.ndarray, budget: int) -> np.ndarray:
    """mode[b, s] = 1 for SLOW, 0 for FAST."""
    B, S = flags.shape
    mode = np.zeros((B, S), np.uint8)
    for b in range(B):
        since = 0
        for s in range(S):
            slow = s == 0 or bool(flags[b, s]) or since == budget
            mode[b, s] = 1 if slow else 0
            since = 0 if slow else since + 1
    return mode


@dataclass
class Plan:
    """Host tables of one trajectory."""
    mode: np.ndarray          # [B, S]
    seq_len: np.ndarray       # [S, B]
    recent_start: np.ndarray  # [S, B] (valid at fast steps)
    keff: np.ndarray = None   # [S, B] selected rows per KV head in the current memory
    slow_ids: List[np.ndarray] = field(default_factory=list)
    fast_ids: List[np.ndarray] = field(default_factory=list)
    max_recent: int = 0


def make_plan(flags: np.ndarray, context: int, budget: int, n_sink: int, n_recent: int,
              top_k: int = 0, sliding: bool = False) -> Plan:
    """Host tables of a trajectory.  The recent segment's left edge is frozen at each slow
    step at max(n_sink, N0 - W), or with `sliding` follows every step at max(n_sink, N - W)."""
    mode = schedule(flags, budget)
    B, S = mode.shape
    seq_len = np.zeros((S, B), np.int32)
    rstart = np.zeros((S, B), np.int32)
    keff = np.zeros((S, B), np.int64)
    max_recent = 1
    cur = np.full(B, n_sink, np.int64)
    cur_k = np.zeros(B, np.int64)
    for s in range(S):
        N = context + s
        seq_len[s, :] = N
        for b in range(B):
            if mode[b, s]:
                # frozen left edge of the recent segment for the following fast steps
                cur[b] = max(n_sink, N - n_recent)
                cur_k[b] = min(top_k, max(0, N - n_recent - n_sink))
            else:
                if sliding:
                    cur[b] = max(n_sink, N - n_recent)
                max_recent = max(max_recent, N - int(cur[b]))
            rstart[s, b] = cur[b]
            keff[s, b] = cur_k[b]
    plan = Plan(mode, seq_len, rstart, keff=keff, max_recent=max_recent)
    for s in range(S):
        plan.slow_ids.append(np.nonzero(mode[:, s])[0].astype(np.int32))
        plan.fast_ids.append(np.nonzero(mode[:, s] == 0)[0].astype(np.int32))
    return plan


# Fewest layers for which a fast step is replayed from a graph (see Engine.enable_graphs).
kGraphMinLayers = 8


def recent_bound(w) -> int:
    """Upper bound of N - recent_start over every fast step of any schedule (see Engine)."""
    return w.n_recent if w.sliding_recent else w.n_recent + w.refresh_budget


def window_query_table(q_all: torch.Tensor, num_kv_heads: int, window: int) -> torch.Tensor:
    """Query layout of windowed slow steps: [S, B, Hkv, window, G, D] (flattened to
    [S, B, Hq * window, D]) with slot k of step s holding the query of step max(0, s - k):
    the current decode query and the ones before it, the first query filling the slots
    before the first step."""
    S, B, Hq, D = q_all.shape
    G = Hq // num_kv_heads
    src = torch.arange(S, device=q_all.device)
    qg = q_all.view(S, B, num_kv_heads, G, D)
    slots = [qg[(src - k).clamp_min(0)] for k in range(window)]
    return torch.stack(slots, dim=3).reshape(S, B, Hq * window, D).contiguous()


class LayerBuffers:
    """Device state of one attention layer."""

    def __init__(self, eng: "Engine", k_cache, v_cache, block_table, q_all):
        w, dev = eng.w, eng.device
        B, Hq, Hkv, D = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
        win = eng.window
        self.k_cache, self.v_cache = k_cache, v_cache
        self.block_table = block_table.to(dev, torch.int32).contiguous()
        self.q_all = q_all                       # [S, B, Hq, D] fp32
        # Slow steps with a query window read q_win[s] [B, Hkv, win, G, D]: slot k holds the
        # query of step max(0, s - k).
        self.q_win = window_query_table(q_all, Hkv, win) if win > 1 else None
        self.key_norm = torch.zeros(B, Hkv, eng.stride, dtype=torch.float32, device=dev)
        self.logits = torch.zeros(B, Hq * win, eng.stride, dtype=torch.float32, device=dev)
        self.lse = torch.zeros(B, Hq * win, dtype=torch.float32, device=dev)
        self.sel_idx = torch.full((B, Hkv, w.top_k), -1, dtype=torch.int32, device=dev)
        dt = k_cache.dtype
        self.packed_k = torch.zeros(B, Hkv, eng.packed_cap, D, dtype=dt, device=dev)
        self.packed_v = torch.zeros(B, Hkv, eng.packed_cap, D, dtype=dt, device=dev)
        self.packed_pos = torch.full((B, Hkv, eng.packed_cap), -1, dtype=torch.int32, device=dev)
        self.packed_len = torch.zeros(B, Hkv, dtype=torch.int32, device=dev)
        self.out = torch.zeros(B, Hq, D, dtype=torch.float32, device=dev)
        self.ev_attn = torch.cuda.Event()
        self.ev_pack = torch.cuda.Event()
        self.pack_pending = False
        self.k_new = self.v_new = None           # [S, B, Hkv, D] (device-controlled steps)
        # slot of every position in the packed buffers, for the incremental pack
        self.slot_map = (torch.full((B, Hkv, eng.stride), -1, dtype=torch.int32, device=dev)
                         if eng._incremental_req is not False else None)


class Engine:
    def __init__(self, w, flags, device="cuda", two_streams: Optional[bool] = None,
                 dbg_scores: bool = False, sel_streams: int = 2,
                 window: Optional[int] = None, device_control: bool = False,
                 tokens=None, boundary_tokens=None, max_recent: Optional[int] = None,
                 full_lists: bool = False, incremental_pack: Optional[bool] = None,
                 paced: Optional[bool] = None, sel_lookahead: Optional[int] = None):
        self.w = w
        self.device = torch.device(device)
        self.device_control = device_control
        # full_lists: every call of a host-scheduled step gets all B slots of its row list
        # (-1 padded), the launch shape of device-controlled steps.
        self.full_lists = full_lists
        # incremental_pack: a slow step copies only the newly selected rows into the packed
        # buffers (sfi_pack_update) instead of all of them (sfi_pack).  None chooses when the
        # stack is known (first step): incremental for several layers, where the pack runs
        # beside the next layer's attention and the bytes it moves slow that attention down;
        # full for one layer, where the pack is on the step's critical path and one kernel
        # beats the update's chain of four short ones (measured both ways on every workload).
        self.incremental_pack = incremental_pack
        self._incremental_req = incremental_pack
        # paced: the host queues a slow step's first Selector-stream wait (on its layer's
        # attention) only once stream 1 has finished every step before the previous one.
        # The host can otherwise run many steps ahead of the GPU, and a wait queued there
        # slowed every kernel on stream 1 meanwhile: fast steps took 0.97 ms instead of
        # 0.89 ms on the 36-layer 128K stack.  One step of lead is kept so that the host's
        # issue of the slow step stays hidden (waiting for the previous step too made slow
        # steps host-bound in a first process on a fresh GPU machine: 6.5 ms instead of 4.8 ms).
        # None chooses by size: paced when a layer's dense K/V per step is at least 8 MiB;
        # below that a step is shorter than its host issue time and the wait costs more than
        # it saves (measured both ways on every workload).
        self.paced = paced
        self._paced_req = paced
        # sel_lookahead k >= 1 (with pacing): layer i's Selector is queued only once stream 1
        # has finished layer i's attention, with k more attention calls queued behind it, so
        # no Selector-stream wait is ever queued ahead of its attention.  None chooses 2 for
        # stacks of more than two layers (measured: 28.9K against 28.7K layer steps/s on the
        # 128K stack, the same for k = 1, 2 and 3) and 0 otherwise, where the host would wait
        # for the step's only attention with nothing queued behind it.
        self.sel_lookahead = sel_lookahead
        self._lookahead_req = sel_lookahead
        # Decode queries pooled into the Selector's evidence at a slow step (1: the current
        # query only).
        self.window = int(w.evidence_window if window is None else window)
        # two_streams: the Selector and pack run on Selector streams beside stream 1's
        # attention (True) or on stream 1 itself (False).  None chooses when the stack is
        # known (first step): Selector streams for several layers, stream 1 for one layer,
        # whose Selector nothing can overlap (the next step's attention reads its pack) and
        # where the cross-stream waits only add latency (measured on every one-layer
        # workload: 8K 49.1K -> 54.0K, 1K 27.5K -> 35.6K, 32K x4 17.8K -> 19.7K, 64K x8
        # 5.40K -> 5.88K layer steps/s).  Device-controlled engines keep their streams.
        self._two_streams_req = two_streams
        two_streams = True if two_streams is None else two_streams
        self.two_streams = two_streams
        flags_np = np.asarray(flags.cpu() if torch.is_tensor(flags) else flags)
        self.plan = make_plan(flags_np, w.context, w.refresh_budget, w.n_sink, w.n_recent,
                              w.top_k, sliding=w.sliding_recent)
        self.shape = L.make_shape(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                  w.pages_per_seq, w.dtype)
        self.params = L.make_params(w.n_sink, w.n_recent, w.top_k, w.nms_radius, w.lam,
                                    w.alpha_soft, w.alpha_cross, w.lambda_clip,
                                    w.nms_greedy)
        self.packed_cap = L.sfi_packed_cap(self.params)
        self.max_len = w.total_len
        self.stride = (self.max_len + 63) // 64 * 64
        # Longest recent segment a fast call can meet.  The host plan knows it; a step decided
        # on the device can only bound it: after a slow step at length N0 the edge is at
        # least N0 - W and at most refresh_budget fast steps follow, so N - edge <= W + budget.
        if max_recent is not None:
            self.max_recent = int(max_recent)
        elif device_control:
            self.max_recent = recent_bound(w)
        else:
            self.max_recent = self.plan.max_recent
        dev = self.device
        S, B = w.steps, w.batch
        self.seq_len_d = torch.from_numpy(self.plan.seq_len).to(dev)
        self.rstart_d = torch.from_numpy(self.plan.recent_start).to(dev)
        slow = np.full((S, B), -1, np.int32)
        fast = np.full((S, B), -1, np.int32)
        for s in range(S):
            slow[s, :len(self.plan.slow_ids[s])] = self.plan.slow_ids[s]
            fast[s, :len(self.plan.fast_ids[s])] = self.plan.fast_ids[s]
        self.slow_ids_d = torch.from_numpy(slow).to(dev)
        self.fast_ids_d = torch.from_numpy(fast).to(dev)
        self.all_ids_d = torch.arange(B, dtype=torch.int32, device=dev)
        # The split plan depends on the number of rows in a call, so size each workspace
        # for the largest requirement over every row count a step can pass.
        win = self.window
        self.ws_slow = L.workspace(max(
            max(L.sfi_slow_attn_ws(self.shape, n, self.max_len),
                L.sfi_slow_attn_window_ws(self.shape, win, n, self.max_len))
            for n in range(1, B + 1)), dev)
        self.ws_fast = L.workspace(
            max(L.sfi_fast_attn_ws(self.shape, n, self.packed_cap, self.max_recent)
                for n in range(1, B + 1)), dev)
        # Selector streams: the Selector and pack of consecutive layers alternate between
        # them, so the dependent kernel chains of two layers run side by side.  Each stream
        # has its own Selector workspace.  The debug score buffer is shared, so with it only
        # one stream is used.
        n_sel = max(1, sel_streams) if (two_streams and not dbg_scores) else 1
        sel_ws = max(L.sfi_select_window_ws(self.shape, self.params, win, n, self.max_len)
                     for n in range(1, B + 1))
        if sel_ws == 0:
            raise ValueError(f"evidence window {win} is not supported for this shape "
                             f"(window >= 1 and group * window <= 16)")
        if incremental_pack is not False:
            sel_ws = max(sel_ws, L.sfi_pack_update_ws(self.shape, self.params, B))
        self.ws_sels = [L.workspace(sel_ws, dev) for _ in range(n_sel)]
        self.ws_sel = self.ws_sels[0]
        self.stream1 = torch.cuda.Stream(device=dev)
        self._sel_streams_own = ([torch.cuda.Stream(device=dev) for _ in range(n_sel)]
                                 if two_streams else [self.stream1])
        self.sel_streams = self._sel_streams_own
        self.stream2 = self.sel_streams[0]
        self.layers: List[LayerBuffers] = []
        if device_control:
            self._init_device_control(tokens, boundary_tokens)
        self.dbg = dbg_scores
        # Device contract flags (sfi_device_status) of every call the engine makes; they stay
        # 0 while the lengths, edges and packed state the engine maintains are consistent.
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.graph = None
        self.graphs = {}
        self._calls = 0
        self.dbg_buf: Optional[torch.Tensor] = None
        if dbg_scores:
            self.dbg_buf = torch.zeros(B, w.num_kv_heads, self.stride, dtype=torch.float32,
                                       device=dev)

    def add_layer(self, k_cache, v_cache, block_table, q_all) -> LayerBuffers:
        lb = LayerBuffers(self, k_cache, v_cache, block_table, q_all)
        n_norm = self.max_len
        if self.device_control:
            # The rows each step appends are taken out of the generated cache and their
            # slots cleared, so the appends must write them back; norms are computed here
            # only for the positions stored before the first step.
            lb.k_new, lb.v_new = self._take_new_rows(lb)
            n_norm = self.n_stored
        # cached key statistic for every stored position (prefill-time work)
        full = torch.full((self.w.batch,), n_norm, dtype=torch.int32, device=self.device)
        # The caches, block table, queries and the buffers above were written on the
        # caller's stream; the engine streams are non-blocking, so order them after it.
        # Stream 2 is ordered behind stream 1 through the per-layer attention events.
        self.stream1.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(self.stream1):
            L.sfi_key_norms(self.shape, lb.k_cache, lb.block_table, full, self.all_ids_d,
                            self.w.batch, 0, n_norm, lb.key_norm, self.stride,
                            stream=self.stream1)
        self.stream1.synchronize()
        self.layers.append(lb)
        return lb

    # ----------------------------------------------------------- on-device step control
    def _init_device_control(self, tokens, boundary_tokens) -> None:
        """State of steps decided on the device: every row stores n_stored = context - 1
        positions before step 0, and step s decodes token tokens[s, b], which joins the
        history (N_s = context + s, as in the host plan)."""
        w, dev = self.w, self.device
        if tokens is None or boundary_tokens is None:
            raise ValueError("device_control needs the decoded tokens and the boundary ids")
        if w.context < 1:
            raise ValueError("device_control needs context >= 1")
        B = w.batch
        self.n_stored = w.context - 1
        self.tokens_d = torch.as_tensor(tokens, dtype=torch.int32).to(dev).contiguous()
        if tuple(self.tokens_d.shape) != (w.steps, B):
            raise ValueError(f"tokens must be [steps, batch] = {(w.steps, B)}")
        self.boundary_d = torch.as_tensor(list(boundary_tokens) or [0],
                                          dtype=torch.int32).to(dev)
        self.n_boundary = len(boundary_tokens)
        # State rows: seq_lens, since_slow, recent_start; state0 holds the values before step
        # 0.  Step s reads the state step s - 1 wrote and writes buffer s % 2 and row lists
        # s % 2, so the Selector and pack of step s - 1, which may still run on their
        # streams, keep reading unchanged lengths and lists.  Step s + 1 cannot overwrite
        # them either: before each layer's attention stream 1 waits for that layer's pack
        # of the step before.
        self.state0 = torch.stack([
            torch.full((B,), self.n_stored, dtype=torch.int32),
            torch.full((B,), -1, dtype=torch.int32),
            torch.zeros(B, dtype=torch.int32)]).to(dev)
        self.state_bufs = [self.state0.clone(), self.state0.clone()]
        self.ws_decode = L.workspace(L.sfi_decode_attn_ws(
            self.shape, self.window, B, self.packed_cap, self.max_recent, self.max_len), dev)
        # row lists [parity][slow, fast][B]
        self.lists = torch.full((2, 2, B), -1, dtype=torch.int32, device=dev)
        self.counts = torch.zeros(2, 2, dtype=torch.int32, device=dev)

    def _take_new_rows(self, lb: LayerBuffers):
        """K/V rows appended at each step, [S, B, Hkv, D]: the generated rows at positions
        N_s - 1 = context + s - 1.  Their cache slots are then zeroed."""
        w = self.w
        S, B = w.steps, w.batch
        pos = torch.arange(S, device=self.device) + (w.context - 1)          # [S]
        pages = lb.block_table[:, pos // w.page_size].t()                     # [S, B]
        slots = (pos % w.page_size)[:, None].expand(S, B)
        k_new = lb.k_cache[pages, :, slots].contiguous()                      # [S, B, Hkv, D]
        v_new = lb.v_cache[pages, :, slots].contiguous()
        lb.k_cache[pages, :, slots] = 0
        lb.v_cache[pages, :, slots] = 0
        return k_new, v_new

    def device_state(self, s: int) -> torch.Tensor:
        """State [3, B] (seq_lens, since_slow, recent_start) written by step s."""
        return self.state_bufs[s % 2]

    def _issue_device_step(self, s: int) -> None:
        """Step s with the slow/fast decision and the K/V append on the device.  Every call
        gets the whole -1-padded row list, so nothing here depends on the decision."""
        w, lib, shp, prm, ok = self.w, self._lib, self._shp, self._prm, self._ok
        B = w.batch
        h1 = self._h1
        s1 = self.stream1
        par = s % 2
        dc = self._dc[par]
        st_in = self._dc_state0 if s == 0 else self._dc[1 - par]["state"]
        sl_p, rs_p = dc["seq_lens"], dc["rstart"]
        slow_p, fast_p = dc["slow"], dc["fast"]
        ws_dec, ws_dec_n = self._ws["decode"]
        win = self.window
        ok("sfi_step_control", lib.sfi_step_control(
            shp, prm, w.refresh_budget, int(w.sliding_recent), self._dc_tok + s * B * 4,
            self._dc_bnd,
            self.n_boundary, st_in, dc["state"], slow_p, fast_p, dc["cnt"], h1))
        for li, lb in enumerate(self.layers):
            P = lb.ptr
            ok("sfi_kv_append", lib.sfi_kv_append(
                shp, P["kn"] + s * lb.kn_step, P["vn"] + s * lb.kn_step, P["k"], P["v"],
                P["bt"], sl_p, self._all_p, B, P["norm"], self.stride, h1))
            if lb.pack_pending:
                s1.wait_event(lb.ev_pack)
                lb.pack_pending = False
            # the fast and the slow rows in one launch pair: one of the two lists is empty
            # at most steps, and its launches would cost as much as a short call
            ok("sfi_decode_attn", lib.sfi_decode_attn(
                shp, win, P["q"] + s * lb.q_step, P["qw"] + s * lb.qw_step, P["pk"], P["pv"],
                P["pl"], self.packed_cap, P["k"], P["v"], P["bt"], rs_p, sl_p, fast_p, slow_p,
                B, self.max_recent, self.max_len, P["out"], P["z"], self.stride, P["lse"],
                self._st, ws_dec, ws_dec_n, h1))
            k = li % len(self.sel_streams)
            s2, h2 = self.sel_streams[k], self._h2[k]
            ws_sel, ws_sel_n = self._ws_sel[k]
            if s2 is not s1:
                lb.ev_attn.record(s1)
                s2.wait_event(lb.ev_attn)
            ok("sfi_select_window", lib.sfi_select_window(
                shp, prm, win, P["z"], self.stride, P["lse"], P["norm"], self.stride, sl_p,
                slow_p, B, self.max_len, P["sel"], self._dbg_p, ws_sel, ws_sel_n, h2))
            self._pack(P, slow_p, B, ws_sel, ws_sel_n, h2)
            if s2 is not s1:
                lb.ev_pack.record(s2)
                lb.pack_pending = True

    def _device_step(self, s: int, timer: Optional[list]) -> None:
        if s == 0:
            # a new trajectory (the last step of the previous one may use state buffer 0)
            self._new_sequences()
        s1 = self.stream1
        e0 = e1 = None
        if timer is not None:
            e0, e1 = self._timing_events()
            e0.record(s1)
        if s in self.graphs:
            self.join()
            with torch.cuda.stream(s1):
                self.graphs[s].replay()
        else:
            self._issue_device_step(s)
        if timer is not None:
            e1.record(s1)
            timer.append(("step", e0, e1, 0, len(self.layers)))

    def enable_device_graphs(self) -> None:
        """Capture every step of a device-controlled trajectory as one HIP graph: the step
        control, and for every layer the append, both attention calls and the Selector and
        pack on their streams (joined back into stream 1 at the end of the graph).  A replay
        needs nothing from the host but the launch.  Call after the last add_layer."""
        if not self.device_control:
            raise RuntimeError("enable_device_graphs needs device_control")
        self._bind()
        self.join()
        self.stream1.wait_stream(torch.cuda.current_stream(self.device))
        torch.cuda.synchronize()
        self.graphs = {}
        pool = None
        for s in range(self.w.steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream1, pool=pool):
                self._issue_device_step(s)
                self.join()
            pool = g.pool()
            self.graphs[s] = g
        self.graph = self.graphs or None
        torch.cuda.synchronize()

    # ------------------------------------------------------------ algorithmic traffic
    def fast_bytes(self, s: int) -> int:
        """Bytes a fast attention call of step s must move: the packed rows and the recent
        window of every fast row (K and V), plus q in and o out (fp32)."""
        w, p = self.w, self.plan
        e = w.elem_bytes
        tot = 0
        for b in p.fast_ids[s]:
            rows = w.n_sink + int(p.keff[s, b]) + int(p.seq_len[s, b] - p.recent_start[s, b])
            tot += w.num_kv_heads * rows * 2 * w.head_dim * e + 8 * w.num_q_heads * w.head_dim
        return tot

    def dense_bytes(self, s: int, ids) -> int:
        """Bytes of dense attention over all N positions of the listed rows."""
        w = self.w
        e = w.elem_bytes
        return sum(w.num_kv_heads * int(self.plan.seq_len[s, b]) * 2 * w.head_dim * e
                   + 8 * w.num_q_heads * w.head_dim for b in ids)

    # ------------------------------------------------------------------------ one step
    def _bind(self) -> None:
        """Cache the ctypes entry points and the raw device pointers step() passes, so a
        step costs one foreign call per kernel launch and no tensor indexing."""
        import ctypes
        self._lib = L.load()
        if self._incremental_req is None:
            self.incremental_pack = len(self.layers) > 1
        if self._paced_req is None:
            w = self.w
            dense = w.batch * w.num_kv_heads * w.context * 2 * w.head_dim * w.elem_bytes
            self.paced = dense >= 8 << 20
        if self._lookahead_req is None:
            self.sel_lookahead = 2 if len(self.layers) > 2 else 0
        if self._two_streams_req is None and not self.device_control:
            self.sel_streams = ([self.stream1] if len(self.layers) == 1
                                else self._sel_streams_own)
            self.stream2 = self.sel_streams[0]
            self.two_streams = self.sel_streams[0] is not self.stream1
        # Start of a step on stream 1, for the pacing of the slow step after it: recorded
        # only at steps followed by a slow step (an event record costs a few microseconds
        # of GPU time, as much as a short fast step's attention), alternating between two.
        self._ev_step = [torch.cuda.Event(), torch.cuda.Event()]
        self._nstep = 0
        self._ev_cur = None   # recorded at the start of the last step issued, or None
        self._ev_prev = None  # recorded at the start of the step before it, or None
        self._has_slow = [bool(x) for x in self.plan.mode.any(axis=0)]
        self._shp = ctypes.byref(self.shape)
        self._prm = ctypes.byref(self.params)
        B = self.w.batch
        self._rowb = B * 4                       # one [B] int32 row of the step tables
        self._seq_len_p = self.seq_len_d.data_ptr()
        self._rstart_p = self.rstart_d.data_ptr()
        self._slow_p = self.slow_ids_d.data_ptr()
        self._fast_p = self.fast_ids_d.data_ptr()
        self._all_p = self.all_ids_d.data_ptr()
        self._h1 = self.stream1.cuda_stream
        self._h2 = [st.cuda_stream for st in self.sel_streams]
        self._ws_sel = [(t.data_ptr(), t.numel()) for t in self.ws_sels]
        self._ws = {k: (t.data_ptr(), t.numel()) for k, t in
                    (("slow", self.ws_slow), ("fast", self.ws_fast))}
        if self.device_control:
            self._ws["decode"] = (self.ws_decode.data_ptr(), self.ws_decode.numel())
        self._dbg_p = self.dbg_buf.data_ptr() if self.dbg_buf is not None else None
        self._st = self.status.data_ptr()
        for lb in self.layers:
            lb.ptr = {k: getattr(lb, a).data_ptr() for k, a in (
                ("k", "k_cache"), ("v", "v_cache"), ("bt", "block_table"), ("q", "q_all"),
                ("norm", "key_norm"), ("z", "logits"), ("lse", "lse"), ("sel", "sel_idx"),
                ("pk", "packed_k"), ("pv", "packed_v"), ("pp", "packed_pos"),
                ("pl", "packed_len"), ("out", "out"))}
            lb.ptr["map"] = lb.slot_map.data_ptr() if lb.slot_map is not None else None
            lb.q_step = lb.q_all[0].numel() * lb.q_all.element_size()
            if lb.k_new is not None:
                lb.ptr["kn"], lb.ptr["vn"] = lb.k_new.data_ptr(), lb.v_new.data_ptr()
                lb.kn_step = lb.k_new[0].numel() * lb.k_new.element_size()
            if lb.q_win is not None:
                lb.ptr["qw"] = lb.q_win.data_ptr()
                lb.qw_step = lb.q_win[0].numel() * lb.q_win.element_size()
            else:
                lb.ptr["qw"], lb.qw_step = lb.ptr["q"], lb.q_step
        if self.device_control:
            self._dc_tok = self.tokens_d.data_ptr()
            self._dc_bnd = self.boundary_d.data_ptr()
            self._dc_state0 = self.state0.data_ptr()
            self._dc = [dict(state=st.data_ptr(), seq_lens=st[0].data_ptr(),
                             rstart=st[2].data_ptr(), slow=self.lists[par, 0].data_ptr(),
                             fast=self.lists[par, 1].data_ptr(),
                             cnt=self.counts[par].data_ptr())
                        for par, st in enumerate(self.state_bufs)]
        self._bound_layers = len(self.layers)

    def enable_graphs(self, min_layers: int = kGraphMinLayers) -> None:
        """Capture, for every step whose rows are all fast, that step's calls of every
        layer as one HIP graph on stream 1 (the step's queries, lengths and recent starts
        are at fixed places in the per-step tables, so each graph holds its own pointers
        and a replay needs no staging).  Call after the last add_layer.

        A graph launch costs more host and device time than issuing a few calls directly
        (measured: about 33 us per replay of a one-layer step against 12 us for its two
        kernels issued back to back), so below `min_layers` layers nothing is captured and
        steps stay call by call."""
        w, dev = self.w, self.device
        if len(self.layers) < min_layers:
            self.graphs, self.graph = {}, None
            return
        self._bind()
        lib, shp = self._lib, self._shp
        B = w.batch
        ws_fast, ws_fast_n = self._ws["fast"]
        self.stream1.wait_stream(torch.cuda.current_stream(dev))
        self.graphs = {}
        pool = None
        for s in range(w.steps):
            if len(self.plan.fast_ids[s]) != B:
                continue
            seq_len = self._seq_len_p + s * self._rowb
            rstart = self._rstart_p + s * self._rowb
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream1, pool=pool):
                for lb in self.layers:
                    P = lb.ptr
                    self._ok("sfi_fast_attn", lib.sfi_fast_attn(
                        shp, P["q"] + s * lb.q_step, P["pk"], P["pv"], P["pl"],
                        self.packed_cap, P["k"], P["v"], P["bt"], rstart, seq_len, self._all_p,
                        B, self.max_recent, P["out"], None, self._st, ws_fast, ws_fast_n,
                        self._h1))
            pool = g.pool()
            self.graphs[s] = g
        self.graph = self.graphs or None
        torch.cuda.synchronize()

    def _pack(self, P, ids, n, ws, ws_n, h) -> None:
        """Pack of one layer: the incremental update, or the full pack."""
        if self.incremental_pack:
            self._ok("sfi_pack_update", self._lib.sfi_pack_update(
                self._shp, self._prm, P["k"], P["v"], P["bt"], P["sel"], ids, n, P["pk"],
                P["pv"], P["pp"], P["pl"], self.packed_cap, P["map"], self.stride, self._st, ws,
                ws_n, h))
        else:
            self._ok("sfi_pack", self._lib.sfi_pack(
                self._shp, self._prm, P["k"], P["v"], P["bt"], P["sel"], ids, n, P["pk"],
                P["pv"], P["pp"], P["pl"], self.packed_cap, h))

    def _new_sequences(self) -> None:
        """Step 0 starts every row afresh: empty the packed buffers (on stream 1), so that the
        trajectory's results do not depend on what an earlier run left in them."""
        self.join()
        if self.incremental_pack:
            with torch.cuda.stream(self.stream1):
                for lb in self.layers:
                    lb.packed_len.zero_()

    @staticmethod
    def _ok(name: str, rc: int) -> None:
        if rc != L.SFI_OK:
            raise L.SfiError(name, rc, L.status_str(rc))

    def step(self, s: int, dense_only: bool = False, timer: Optional[list] = None,
             time_every: int = 1) -> None:
        """Issue decode step s of every layer (no host synchronisation).

        dense_only runs the Full-KV baseline: dense attention for every sequence, no
        Selector, no logits.  When `timer` is a list, every `time_every`-th attention call
        (counted over the engine's life) is bracketed by two events on stream 1 and
        (kind, start, end, algorithmic bytes, calls) is appended; graph replays are sampled the
        same way, each bracketed as a whole (calls = layers).
        """
        if getattr(self, "_bound_layers", -1) != len(self.layers):
            self._bind()
        if self.device_control and not dense_only:
            self._device_step(s, timer)
            return
        if not dense_only:
            self._ev_prev = self._ev_cur
            self._ev_cur = None
            nxt = (s + 1) % self.w.steps
            if self.paced and self._has_slow[nxt] and self.sel_streams[0] is not self.stream1:
                self._ev_cur = self._ev_step[self._nstep % 2]
                self._ev_cur.record(self.stream1)
                self._nstep += 1
        if s == 0 and not dense_only:
            self._new_sequences()
        # The graph waits for every layer's pending pack before its first call, so the
        # first fast step after a slow step is issued call by call: its layer i then waits
        # only for layer i's pack and overlaps the Selector work still queued on stream 2.
        if self.graph is not None and not dense_only and s in self.graphs and \
                not any(lb.pack_pending for lb in self.layers):
            self._step_graph(s, timer, time_every)
            return
        w, lib, shp, prm = self.w, self._lib, self._shp, self._prm
        n_slow = len(self.plan.slow_ids[s])
        n_fast = len(self.plan.fast_ids[s])
        # rows each call is given (its list is -1 padded past the listed rows)
        m_slow = w.batch if self.full_lists else n_slow
        m_fast = w.batch if self.full_lists else n_fast
        seq_len = self._seq_len_p + s * self._rowb
        rstart = self._rstart_p + s * self._rowb
        slow_ids = self._slow_p + s * self._rowb
        fast_ids = self._fast_p + s * self._rowb
        s1 = self.stream1
        h1 = self._h1
        ws_slow, ws_slow_n = self._ws["slow"]
        ws_fast, ws_fast_n = self._ws["fast"]
        ok = self._ok
        win = self.window

        def timed(li, kind, nbytes, fn):
            # every time_every-th call of the engine's life is timed (a global count, so
            # one-layer stacks are sampled as sparsely as deep ones)
            self._calls += 1
            if timer is None or (self._calls - 1) % time_every:
                fn()
                return
            e0, e1 = self._timing_events()
            e0.record(s1)
            fn()
            e1.record(s1)
            timer.append((kind, e0, e1, nbytes, 1))

        fb = self.fast_bytes(s) if (timer is not None and n_fast) else 0
        db = self.dense_bytes(s, range(w.batch) if dense_only else self.plan.slow_ids[s]) \
            if timer is not None else 0

        def selector(li, lb, P, recorded=False, host_wait=False):
            """Selector and pack of layer li on its Selector stream, behind its attention.
            recorded: the attention event is already recorded; host_wait: the host first
            waits for it."""
            k = li % len(self.sel_streams)
            s2, h2 = self.sel_streams[k], self._h2[k]
            ws_sel, ws_sel_n = self._ws_sel[k]
            if s2 is not s1:
                if not recorded:
                    lb.ev_attn.record(s1)
                if host_wait:
                    lb.ev_attn.synchronize()
                if pace and not paced_wait[0]:
                    # stream 1 has finished every step before the previous one; the previous
                    # step and this step's first attention keep the GPU busy meanwhile
                    if self._ev_prev is not None:
                        self._ev_prev.synchronize()
                    paced_wait[0] = True
                s2.wait_event(lb.ev_attn)
            ok("sfi_select_window", lib.sfi_select_window(
                shp, prm, win, P["z"], self.stride, P["lse"], P["norm"], self.stride, seq_len,
                slow_ids, m_slow, self.max_len, P["sel"], self._dbg_p, ws_sel, ws_sel_n, h2))
            self._pack(P, slow_ids, m_slow, ws_sel, ws_sel_n, h2)
            if s2 is not s1:
                lb.ev_pack.record(s2)
                lb.pack_pending = True

        # Pacing (see `paced`): the first Selector-stream wait of a slow step is queued only
        # once stream 1 has finished the steps before the previous one.
        pace = bool(n_slow) and not dense_only and self.paced and self.sel_streams[0] is not s1
        paced_wait = [False]
        pending = []
        for li, lb in enumerate(self.layers):
            P = lb.ptr
            q = P["q"] + s * lb.q_step
            if dense_only:
                timed(li, "dense", db, lambda: ok("sfi_slow_attn", lib.sfi_slow_attn(
                    shp, q, P["k"], P["v"], P["bt"], seq_len, self._all_p, w.batch,
                    self.max_len, P["out"], None, 0, P["lse"], self._st, ws_slow, ws_slow_n,
                    h1)))
                continue
            if lb.pack_pending:
                s1.wait_event(lb.ev_pack)
                lb.pack_pending = False
            if n_fast:
                timed(li, "fast", fb, lambda: ok("sfi_fast_attn", lib.sfi_fast_attn(
                    shp, q, P["pk"], P["pv"], P["pl"], self.packed_cap, P["k"], P["v"],
                    P["bt"], rstart, seq_len, fast_ids, m_fast, self.max_recent, P["out"],
                    None, self._st, ws_fast, ws_fast_n, h1)))
            if n_slow:
                qw = P["qw"] + s * lb.qw_step
                timed(li, "slow", db, lambda: ok(
                    "sfi_slow_attn_window", lib.sfi_slow_attn_window(
                        shp, win, qw, P["k"], P["v"], P["bt"], seq_len, slow_ids, m_slow,
                        self.max_len, P["out"], P["z"], self.stride, P["lse"], self._st,
                        ws_slow, ws_slow_n, h1)))
                if pace and self.sel_lookahead > 0:
                    lb.ev_attn.record(s1)
                    pending.append((li, lb, P))
                    while pending and pending[0][0] <= li - self.sel_lookahead:
                        lj, lbj, Pj = pending.pop(0)
                        selector(lj, lbj, Pj, recorded=True, host_wait=True)
                else:
                    selector(li, lb, P)
        # The last layers' Selectors are queued at once: their waits sit behind at most
        # sel_lookahead attention calls, and the host goes on to the next step meanwhile.
        for lj, lbj, Pj in pending:
            selector(lj, lbj, Pj, recorded=True)

    def _step_graph(self, s: int, timer: Optional[list], time_every: int = 1) -> None:
        """Fast step s of every row through its captured graph (no pack pending).  With a
        timer, every time_every-th replay (counted over the engine's life) is bracketed."""
        s1 = self.stream1
        g = self.graphs[s]
        self._replays = getattr(self, "_replays", 0) + 1
        with torch.cuda.stream(s1):
            if timer is None or (self._replays - 1) % max(1, time_every):
                g.replay()
            else:
                e0, e1 = self._timing_events()
                e0.record(s1)
                g.replay()
                e1.record(s1)
                nl = len(self.layers)
                timer.append(("fast", e0, e1, self.fast_bytes(s) * nl, nl))

    def reserve_timing_events(self, n: int) -> None:
        """Create n pairs of timing events now, for the timed calls to take: event creation
        can cost milliseconds of host time in a fresh process, which a timed region should
        not include."""
        self._ev_pool = [(torch.cuda.Event(enable_timing=True),
                          torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    def _timing_events(self):
        pool = getattr(self, "_ev_pool", None)
        if pool:
            return pool.pop()
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def join(self) -> None:
        """Make stream 1 wait for every outstanding Selector/pack."""
        for lb in self.layers:
            if lb.pack_pending:
                self.stream1.wait_event(lb.ev_pack)
                lb.pack_pending = False

    def device_status(self) -> int:
        """The contract flags the engine's calls reported so far (waits for the device)."""
        self.join()
        torch.cuda.synchronize(self.device)
        return int(self.status.item())

    def mode(self, s: int) -> np.ndarray:
        return self.plan.mode[:, s]
