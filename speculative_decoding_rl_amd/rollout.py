"""Python face of the rollout C ABI: argument marshalling around libsdrl.so.

PyTorch supplies device memory (the arena, the target weights) and the
stream; every step of the method runs in the library's kernels.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib
from ._lib import check


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_lib.I32P)


class Engine:
    """One rollout context (er_ctx) over a model's weights.

    shape: object with n_layers, d_model, n_q_heads, n_kv_heads, head_dim,
    ffn, vocab, dtype ('bf16'|'f32'), rms_eps, rope_theta.
    weights: name -> torch tensor on the GPU (names as in synth.tensor_shapes).
    """

    def __init__(self, shape, weights: dict, quant: str = "w4", *, seed: int = 0, temperature: float = 1.0,
                 top_p: float = 1.0, gamma_init: int = 4, gamma_min: int = 1, gamma_max: int = 8,
                 ema_beta: float = 0.3, switch_margin: float = 1.02, alpha_init: float = 0.8,
                 policy: int = _lib.ER_POLICY_AUTO, max_seqs: int = 64, max_batch: int = 64, max_ctx: int = 4096,
                 prefill_chunk: int = 4096, kv_blocks: int = 0, arena_bytes: int | None = None,
                 hbm_bytes_per_s: float = 0.0, flops_per_s: float = 0.0, t_fwd_s: float = -1.0,
                 quant_lm_head: bool = True, device=None, stream=None):
        import torch

        self.lib = _lib.load()
        self.shape = shape
        self.md = _lib.ModelDesc(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                                 shape.ffn, shape.vocab, _lib.ER_BF16 if shape.dtype == "bf16" else _lib.ER_F32,
                                 shape.rms_eps, shape.rope_theta)
        self.dd = _lib.DraftDesc(_lib.ER_W4_G128_ASYM if quant == "w4" else _lib.ER_W8_PERCH_SYM, 128,
                                 1 if quant_lm_head else 0)
        self.rd = _lib.RolloutDesc(seed, temperature, top_p, gamma_init, gamma_min, gamma_max, ema_beta,
                                   switch_margin, alpha_init, policy, 16, max_seqs, max_batch, max_ctx,
                                   prefill_chunk, kv_blocks, hbm_bytes_per_s, flops_per_s, t_fwd_s)
        self.gamma_max = gamma_max
        self.vocab = shape.vocab
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        if arena_bytes is None:
            need = C.c_size_t(0)
            check(self.lib.er_arena_bytes(C.byref(self.md), C.byref(self.dd), C.byref(self.rd), max(kv_blocks, 1),
                                          C.byref(need)), None, "er_arena_bytes")
            arena_bytes = int(need.value)
        self.arena = torch.empty(arena_bytes, dtype=torch.uint8, device=dev)
        self._set_weight_struct(weights)
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        ctx = C.c_void_p()
        rc = self.lib.er_rollout_init(C.byref(self.md), C.byref(self.ws), C.byref(self.dd), C.byref(self.rd),
                                      C.c_void_p(self.arena.data_ptr()), arena_bytes,
                                      C.c_void_p(self.stream.cuda_stream), C.byref(ctx))
        self.ctx = ctx
        if rc != 0:
            msg = self.lib.er_last_error(ctx).decode() if ctx else ""
            if ctx:
                self.lib.er_destroy(ctx)
                self.ctx = None
            raise _lib.ErError(rc, f"er_rollout_init: {msg}")

    def _set_weight_struct(self, weights):
        L = self.shape.n_layers
        self.weights = weights  # keep alive
        arr = lambda key: (C.c_void_p * L)(*[weights[f"{key}.{l}"].data_ptr() for l in range(L)])
        self._arrs = {k: arr(k) for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgate_up", "wdown")}
        cast = lambda a: C.cast(a, C.POINTER(C.c_void_p))
        self.ws = _lib.Weights(weights["embed"].data_ptr(), weights["final_norm"].data_ptr(),
                               weights["lm_head"].data_ptr(), cast(self._arrs["attn_norm"]), cast(self._arrs["wqkv"]),
                               cast(self._arrs["wo"]), cast(self._arrs["mlp_norm"]), cast(self._arrs["wgate_up"]),
                               cast(self._arrs["wdown"]))

    # ---- lifecycle ----------------------------------------------------------
    def close(self):
        if getattr(self, "ctx", None):
            self.lib.er_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def update_weights(self, weights: dict):
        self._set_weight_struct(weights)
        check(self.lib.er_update_weights(self.ctx, C.byref(self.ws)), self.ctx, "er_update_weights")

    # ---- sequences ------------------------------------------------------------
    def kv_alloc(self, prompt_lens, max_new, share_group=None) -> np.ndarray:
        pl, mn = _i32(prompt_lens), _i32(max_new)
        n = len(pl)
        ids = np.zeros(n, dtype=np.int32)
        sg = _p32(_i32(share_group)) if share_group is not None else None
        if share_group is not None:
            sgarr = _i32(share_group)
            sg = _p32(sgarr)
        check(self.lib.er_kv_alloc(self.ctx, n, _p32(pl), _p32(mn), sg, _p32(ids)), self.ctx, "er_kv_alloc")
        return ids

    def kv_fork(self, parent: int, max_new) -> np.ndarray:
        """Children of a running sequence sharing its committed KV (copy-on-write at the last block)."""
        mn = _i32(max_new)
        out = np.zeros(len(mn), dtype=np.int32)
        check(self.lib.er_kv_fork(self.ctx, int(parent), len(mn), _p32(mn), _p32(out)), self.ctx, "er_kv_fork")
        return out

    def prefill(self, ids, prompts) -> np.ndarray:
        ids = _i32(ids)
        toks = _i32(np.concatenate([np.asarray(p, dtype=np.int32).ravel() for p in prompts]))
        offs = np.zeros(len(prompts) + 1, dtype=np.int64)
        offs[1:] = np.cumsum([len(np.asarray(p).ravel()) for p in prompts])
        out = np.zeros(len(ids), dtype=np.int32)
        check(self.lib.er_prefill(self.ctx, len(ids), _p32(ids), _p32(toks), offs.ctypes.data_as(_lib.I64P), _p32(out)),
              self.ctx, "er_prefill")
        return out

    def set_history(self, hist, gamma: int = 4, max_batch: int = 64):
        """Attach a History (drafts copied from earlier rollouts); None detaches."""
        check(self.lib.er_set_history(self.ctx, hist.h if hist is not None else None, gamma, max_batch), self.ctx,
              "er_set_history")
        self._hist = hist   # keep the cache alive while attached

    def history_step(self, ids):
        ids = _i32(ids)
        n = len(ids)
        tok = np.zeros((n, self.gamma_max + 1), dtype=np.int32)
        ne = np.zeros(n, dtype=np.int32)
        info = _lib.StepInfo()
        check(self.lib.er_history_step(self.ctx, n, _p32(ids), _p32(tok), _p32(ne), C.byref(info)), self.ctx,
              "er_history_step")
        return tok, ne, info

    def spec_step(self, ids):
        ids = _i32(ids)
        n = len(ids)
        tok = np.zeros((n, self.gamma_max + 1), dtype=np.int32)
        ne = np.zeros(n, dtype=np.int32)
        info = _lib.StepInfo()
        check(self.lib.er_spec_step(self.ctx, n, _p32(ids), _p32(tok), _p32(ne), C.byref(info)), self.ctx,
              "er_spec_step")
        return tok, ne, info

    def ar_step(self, ids):
        ids = _i32(ids)
        n = len(ids)
        tok = np.zeros(n, dtype=np.int32)
        info = _lib.StepInfo()
        check(self.lib.er_ar_step(self.ctx, n, _p32(ids), _p32(tok), C.byref(info)), self.ctx, "er_ar_step")
        return tok, info

    def step(self, ids):
        ids = _i32(ids)
        n = len(ids)
        tok = np.zeros((n, self.gamma_max + 1), dtype=np.int32)
        ne = np.zeros(n, dtype=np.int32)
        info = _lib.StepInfo()
        check(self.lib.er_step(self.ctx, n, _p32(ids), _p32(tok), _p32(ne), C.byref(info)), self.ctx, "er_step")
        return tok, ne, info

    def rollout(self, ids, cap: int):
        ids = _i32(ids)
        n = len(ids)
        out = np.zeros((n, cap), dtype=np.int32)
        lens = np.zeros(n, dtype=np.int32)
        st = _lib.Stats()
        check(self.lib.er_rollout(self.ctx, n, _p32(ids), cap, _p32(out), _p32(lens), C.byref(st)), self.ctx,
              "er_rollout")
        return out, lens, st.as_dict()

    def set_gamma(self, g: int):
        check(self.lib.er_set_gamma(self.ctx, g), self.ctx, "er_set_gamma")

    def set_policy(self, p: int):
        check(self.lib.er_set_policy(self.ctx, p), self.ctx, "er_set_policy")

    def kv_free(self, ids):
        ids = _i32(ids)
        check(self.lib.er_kv_free(self.ctx, len(ids), _p32(ids)), self.ctx, "er_kv_free")

    def seq_info(self, sid: int):
        g, c, f = C.c_int32(), C.c_int32(), C.c_int32()
        check(self.lib.er_seq_info(self.ctx, sid, C.byref(g), C.byref(c), C.byref(f)), self.ctx, "er_seq_info")
        return g.value, c.value, bool(f.value)

    def stats(self) -> dict:
        st = _lib.Stats()
        check(self.lib.er_get_stats(self.ctx, C.byref(st)), self.ctx, "er_get_stats")
        return st.as_dict()

    def reset_stats(self):
        check(self.lib.er_reset_stats(self.ctx), self.ctx, "er_reset_stats")

    def cost_model(self) -> dict:
        m = _lib.CostModel()
        check(self.lib.er_get_cost_model(self.ctx, C.byref(m)), self.ctx, "er_get_cost_model")
        return {f: getattr(m, f) for f, _ in m._fields_}

    def plan_state(self) -> dict:
        """State of the roofline policy (last choice, AR streak, probe gap)."""
        st = _lib.PlanState()
        check(self.lib.er_get_plan_state(self.ctx, C.byref(st)), self.ctx, "er_get_plan_state")
        return dict(choice=st.choice, ar_streak=st.ar_streak, probe_every=st.probe_every)

    def guard(self) -> dict:
        """State of the measured-timing guard (policy ER_POLICY_TIMING)."""
        g = _lib.GuardState()
        check(self.lib.er_get_guard(self.ctx, C.byref(g)), self.ctx, "er_get_guard")
        return dict(step=g.step, ema_ar=list(g.ema_ar), ema_sd=list(g.ema_sd), n_ar=list(g.n_ar),
                    probe_left=list(g.probe_left), cool_until=list(g.cool_until), cool_len=list(g.cool_len))

    def set_persistent(self, on: bool):
        """Run forwards of <= 16 rows as one persistent launch (bf16 models; off by default)."""
        check(self.lib.er_set_persistent(self.ctx, int(bool(on))), self.ctx, "er_set_persistent")

    def set_graphs(self, max_batch: int):
        """Replay recorded graphs for steps of at most max_batch sequences (0: off, the default)."""
        check(self.lib.er_set_graphs(self.ctx, int(max_batch)), self.ctx, "er_set_graphs")

    def set_library_gemm(self, min_rows: int):
        """Run the target's projections as hipBLASLt GEMMs: -1 from each shape's measured row threshold
        (the default), > 0 from min_rows rows for every shape, 0 never."""
        check(self.lib.er_set_library_gemm(self.ctx, int(min_rows)), self.ctx, "er_set_library_gemm")

    def graph_stats(self) -> dict:
        g = _lib.GraphStats()
        check(self.lib.er_get_graph_stats(self.ctx, C.byref(g)), self.ctx, "er_get_graph_stats")
        return {f: getattr(g, f) for f, _ in g._fields_}

    def set_decode_spin_limit(self, polls: int):
        check(self.lib.er_set_decode_spin_limit(self.ctx, int(polls)), self.ctx, "er_set_decode_spin_limit")

    def set_decode_trace(self, on: bool):
        check(self.lib.er_set_decode_trace(self.ctx, int(bool(on))), self.ctx, "er_set_decode_trace")

    def decode_trace(self):
        """(work_us, release_us) per phase of the last traced persistent forward."""
        w = (C.c_double * 1024)()
        r = (C.c_double * 1024)()
        n = C.c_int()
        check(self.lib.er_get_decode_trace(self.ctx, w, r, 1024, C.byref(n)), self.ctx, "er_get_decode_trace")
        return np.array(w[:n.value]), np.array(r[:n.value])

    def persistent(self) -> bool:
        v = C.c_int()
        check(self.lib.er_get_persistent(self.ctx, C.byref(v)), self.ctx, "er_get_persistent")
        return bool(v.value)

    def set_fused(self, on: bool):
        check(self.lib.er_set_fused(self.ctx, int(bool(on))), self.ctx, "er_set_fused")

    def set_timing(self, period: int, first_n: int = 0):
        check(self.lib.er_set_timing(self.ctx, period, first_n), self.ctx, "er_set_timing")

    def free_blocks(self):
        f, t = C.c_int64(), C.c_int64()
        check(self.lib.er_kv_free_blocks(self.ctx, C.byref(f), C.byref(t)), self.ctx, "er_kv_free_blocks")
        return f.value, t.value

    def set_kernel_profile(self, on):
        """on: False/True, or _lib.ER_KPROF_ATTENTION (attention launches only)."""
        mode = on if isinstance(on, int) and not isinstance(on, bool) else (_lib.ER_KPROF_ALL if on else _lib.ER_KPROF_OFF)
        check(self.lib.er_set_kernel_profile(self.ctx, mode), self.ctx, "er_set_kernel_profile")

    def reset_kernel_profile(self):
        check(self.lib.er_reset_kernel_profile(self.ctx), self.ctx, "er_reset_kernel_profile")

    def kernel_profile(self) -> list:
        n = C.c_int()
        check(self.lib.er_get_kernel_profile(self.ctx, None, 0, C.byref(n)), self.ctx, "er_get_kernel_profile")
        arr = (_lib.KernelStat * max(1, n.value))()
        check(self.lib.er_get_kernel_profile(self.ctx, arr, n.value, C.byref(n)), self.ctx, "er_get_kernel_profile")
        return [dict(name=a.name.decode(), launches=a.launches, ms=a.ms, bytes=a.bytes, flops=a.flops)
                for a in arr[:n.value]]

    def debug_logits(self, which: int, slot: int) -> np.ndarray:
        rows = C.c_int32()
        check(self.lib.er_debug_logits(self.ctx, which, slot, None, C.byref(rows)), self.ctx, "er_debug_logits")
        out = np.zeros((rows.value, self.vocab), dtype=np.float32)
        check(self.lib.er_debug_logits(self.ctx, which, slot, out.ctypes.data_as(C.POINTER(C.c_float)),
                                       C.byref(rows)), self.ctx, "er_debug_logits")
        return out

    def debug_drafts(self, batch: int, gamma: int) -> np.ndarray:
        out = np.zeros((batch, gamma), dtype=np.int32)
        check(self.lib.er_debug_drafts(self.ctx, _p32(out)), self.ctx, "er_debug_drafts")
        return out


def controller_choose(cost: dict, batch: int, mean_ctx: float, alpha: float, gamma_min: int, gamma_max: int,
                      current: int = -1, margin: float = 1.02) -> int:
    lib = _lib.load()
    m = _lib.CostModel(**cost)
    g = C.c_int()
    check(lib.er_controller_choose(C.byref(m), batch, mean_ctx, alpha, gamma_min, gamma_max, current, margin,
                                   C.byref(g)), None, "er_controller_choose")
    return g.value


def controller_times(cost: dict, batch: int, mean_ctx: float, gamma: int):
    """(AR step time, SD step time at gamma) of the library's cost model."""
    lib = _lib.load()
    m = _lib.CostModel(**cost)
    ta, ts = C.c_double(), C.c_double()
    check(lib.er_controller_times(C.byref(m), batch, mean_ctx, gamma, C.byref(ta), C.byref(ts)), None,
          "er_controller_times")
    return ta.value, ts.value


def controller_plan(cost: dict, state: dict, policy: int, batch: int, mean_ctx: float, alpha_ema: float,
                    alpha_init: float, gamma_lo: int, gamma_hi: int, margin: float = 1.02) -> int:
    """One step of the library's roofline policy; `state` (choice, ar_streak, probe_every) is updated in place."""
    lib = _lib.load()
    m = _lib.CostModel(**cost)
    st = _lib.PlanState(state["choice"], state["ar_streak"], state["probe_every"])
    g = C.c_int()
    check(lib.er_controller_plan(C.byref(m), C.byref(st), policy, batch, mean_ctx, alpha_ema, alpha_init, gamma_lo,
                                 gamma_hi, margin, C.byref(g)), None, "er_controller_plan")
    state.update(choice=st.choice, ar_streak=st.ar_streak, probe_every=st.probe_every)
    return g.value


class History:
    """The model-free history drafter's cache (er_history_*): records of earlier rollouts."""

    def __init__(self, prefix_len: int = 2):
        self.lib = _lib.load()
        h = C.c_void_p()
        check(self.lib.er_history_create(prefix_len, C.byref(h)), None, "er_history_create")
        self.h = h

    def add(self, prompt, response, reward: float = 0.0):
        p, r = _i32(prompt), _i32(response)
        check(self.lib.er_history_add(self.h, len(p), _p32(p), len(r), _p32(r), float(reward)), None,
              "er_history_add")

    def propose(self, prompt, context, gamma: int) -> list:
        p, c = _i32(prompt), _i32(context)
        out = np.zeros(max(1, gamma), dtype=np.int32)
        n = np.zeros(1, dtype=np.int32)
        check(self.lib.er_history_propose(self.h, len(p), _p32(p), len(c), _p32(c), gamma, _p32(out), _p32(n)), None,
              "er_history_propose")
        return [int(t) for t in out[:int(n[0])]]

    def records(self) -> int:
        n = C.c_int64()
        check(self.lib.er_history_records(self.h, C.byref(n)), None, "er_history_records")
        return int(n.value)

    def close(self):
        if self.h:
            self.lib.er_history_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
