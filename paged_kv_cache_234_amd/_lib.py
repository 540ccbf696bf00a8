"""ctypes binding of libpagedattn.so (the C ABI declared in include/pa.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks their shapes/dtypes against each other, and passes
raw device pointers and sizes to the C entry point of the same name.  All
work runs in the HIP kernels; there is no fallback.  A missing or unloadable
library raises immediately.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_DT_F32, PA_DT_BF16, PA_DT_FP8_E4M3 = 0, 1, 2
PA_OK, PA_ERR_ARG, PA_ERR_UNSUPPORTED, PA_ERR_LAUNCH, PA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
BLOCK_SIZE = 16

EXPORTED = (
    "pa_kv_append", "pa_decode", "pa_decode_append", "pa_decode_cascade", "pa_decode_multi",
    "pa_decode_splitk_reduce", "pa_prefill_chunk", "pa_decode_plan", "pa_decode_plan_bytes",
    "pa_status_string", "pa_decode_workspace_bytes", "pa_selftest", "pa_decode_noalloc",
    "pa_decode_noalloc_max_bytes", "pa_read_probe",
)

_lib = None


class PAError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__("%s failed: %s (status %d)" % (fn, text, status))
        self.status = status


def load(path=LIB_PATH):
    """Load the library once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libpagedattn.so not built (%s); run "
                           "`python -m paged_kv_cache_234_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, f32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    lib.pa_kv_append.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, st]
    lib.pa_decode.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                              f32, i32, i32, vp, vp, vp, st]
    lib.pa_decode_append.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, i32,
                                     i32, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp,
                                     ctypes.c_size_t, st]
    lib.pa_decode_plan.argtypes = [vp, ctypes.c_size_t, i32, vp, i32, vp, i32, vp, vp, vp, vp, i32,
                                   i32, vp, i32, i32, i32, i32, i32, i32, i32, st]
    lib.pa_decode_plan_bytes.argtypes = [i32, i32, i32]
    lib.pa_decode_plan_bytes.restype = ctypes.c_size_t
    lib.pa_decode_cascade.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, i32,
                                      vp, vp, vp,
                                      i32, i32, i32, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp,
                                      ctypes.c_size_t, st]
    lib.pa_decode_multi.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp, vp, i32, vp, vp, vp, i32,
                                    vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp,
                                    ctypes.c_size_t, st]
    lib.pa_decode_splitk_reduce.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, st]
    lib.pa_prefill_chunk.argtypes = [vp, vp, i32, vp, i32, i32, vp, vp, i32, vp, vp, vp, i32, vp,
                                     i32, i32, i32, i32, f32, st]
    lib.pa_status_string.argtypes = [i32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_selftest.argtypes = []
    lib.pa_decode_noalloc.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, i32, i32, i32,
                                      i32, i32, f32, i32, i32, st]
    lib.pa_read_probe.argtypes = [vp, ctypes.c_size_t, vp, i32, vp, ctypes.c_size_t, st]
    lib.pa_read_probe.restype = ctypes.c_int
    lib.pa_decode_noalloc_max_bytes.argtypes = []
    lib.pa_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    for fn in ("pa_kv_append", "pa_decode", "pa_decode_append", "pa_decode_cascade",
               "pa_decode_multi", "pa_decode_splitk_reduce", "pa_prefill_chunk", "pa_decode_plan",
               "pa_selftest", "pa_decode_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status):
    return load().pa_status_string(int(status)).decode()


def _check(fn, status):
    if status != PA_OK:
        raise PAError(fn, status, status_string(status))


def _dt(t):
    if t.dtype == torch.float32:
        return PA_DT_F32
    if t.dtype == torch.bfloat16:
        return PA_DT_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_DT_FP8_E4M3
    raise TypeError("unsupported tensor dtype %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t, name):
    if t.dtype != torch.int32:
        raise TypeError("%s must be int32" % name)
    return _ptr(t)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _pool_dims(k_cache, v_cache):
    """K [NB, Hkv, D/X, bs, X] (X = 16 bytes of elements), V [NB, Hkv, D, bs]."""
    if k_cache.dim() != 5:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, head_dim/X, block_size, X]")
    nb, hkv, dx, bs, x = k_cache.shape
    if x * k_cache.element_size() != 16:
        raise ValueError("k_cache's last dimension must hold 16 bytes")
    d = dx * x
    if tuple(v_cache.shape) != (nb, hkv, d, bs) or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, head_dim, block_size] "
                         "of k_cache's dtype")
    return nb, hkv, bs, d


def pa_selftest():
    _check("pa_selftest", load().pa_selftest())


def pa_decode_workspace_bytes(batch, num_heads, head_dim, max_partitions):
    return int(load().pa_decode_workspace_bytes(batch, num_heads, head_dim, max_partitions))


def pa_decode_plan_bytes(rows, k_cache, head_dim):
    """Bytes of a launch plan for `rows` rows (the batch, plus the prefix
    groups for the cascade) over pools of k_cache's dtype."""
    return int(load().pa_decode_plan_bytes(int(rows), _dt(k_cache), int(head_dim)))


def decode_plan_buffer(rows, k_cache, head_dim, device="cuda"):
    """An int32 device buffer large enough for pa_decode_plan."""
    n = -(-pa_decode_plan_bytes(rows, k_cache, head_dim) // 4)
    return torch.empty(max(n, 1), dtype=torch.int32, device=device)


def _plan_ptr(plan):
    if plan is None:
        return None
    if plan.dtype != torch.int32:
        raise TypeError("plan must be int32")
    return _ptr(plan)


def _plan_bytes(plan):
    return 0 if plan is None else plan.numel() * 4


PA_PLAN_DECODE_APPEND, PA_PLAN_DECODE_CASCADE, PA_PLAN_DECODE_MULTI = 0, 1, 2


def pa_decode_plan(plan, block_tables, context_lens, num_heads, k_cache, v_cache, partition_size=0,
                   max_partitions=1, groups=None, queries=None, new_slots=None, stream=None):
    """Fill `plan` (from decode_plan_buffer) with the decode prologue of this
    batch for launches with the same arguments: pa_decode_append by default;
    pa_decode_cascade with groups=(group_start, group_seqs, group_prefix_lens,
    max_group_size); pa_decode_multi with queries=(query_start_loc,
    max_query_len).  new_slots: the slots the launches will append with."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    B = context_lens.numel()
    if block_tables.shape[0] != B:
        raise ValueError("inconsistent decode shapes")
    entry, gs, gq, gp, ng, mg, qsl, mq = PA_PLAN_DECODE_APPEND, None, None, None, 0, 0, None, 0
    if groups is not None:
        entry = PA_PLAN_DECODE_CASCADE
        gs, gq, gp, mg = groups
        ng = gs.numel() - 1
        gs, gq, gp = (_i32(gs, "group_start"), _i32(gq, "group_seqs"),
                      _i32(gp, "group_prefix_lens"))
    elif queries is not None:
        entry = PA_PLAN_DECODE_MULTI
        qsl, mq = queries
        qsl = _i32(qsl, "query_start_loc")
    st = load().pa_decode_plan(_plan_ptr(plan), _plan_bytes(plan), entry,
                               _i32(block_tables, "block_tables"), block_tables.shape[1],
                               _i32(context_lens, "context_lens"), B,
                               None if new_slots is None else _i32(new_slots, "new_slots"),
                               gs, gq, gp, ng, int(mg), qsl,
                               int(mq), int(num_heads), hkv, d, _dt(k_cache), int(partition_size),
                               int(max_partitions), _stream(stream))
    _check("pa_decode_plan", st)


def pa_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale=None, v_scale=None,
                 stream=None):
    """k_new, v_new [T, Hkv, D]; pools as in include/pa.h; slot_mapping int32 [T]."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    T = k_new.shape[0]
    if tuple(k_new.shape) != (T, hkv, d) or tuple(v_new.shape) != (T, hkv, d):
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have one entry per token")
    st = load().pa_kv_append(_ptr(k_new), _ptr(v_new), _dt(k_new), _ptr(k_cache), _ptr(v_cache),
                             _dt(k_cache), _ptr(k_scale), _ptr(v_scale),
                             _i32(slot_mapping, "slot_mapping"), T, nb, hkv, d, bs,
                             _stream(stream))
    _check("pa_kv_append", st)


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=None,
              v_scale=None, partition_size=0, max_partitions=1, part_max=None, part_sum=None,
              part_out=None, stream=None):
    """out, q [B, Hq, D]; block_tables int32 [B, W]; context_lens int32 [B]."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    B, hq = q.shape[0], q.shape[1]
    if q.shape[2] != d or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent decode shapes")
    if partition_size > 0:
        want = (B, hq, max_partitions)
        for t in (part_max, part_sum):
            if t is None or tuple(t.shape) != want or t.dtype != torch.float32:
                raise ValueError("part_max/part_sum must be float32 %s" % (want,))
        if part_out is None or tuple(part_out.shape) != want + (d,):
            raise ValueError("part_out must be float32 %s" % (want + (d,),))
    elif out is None or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    st = load().pa_decode(_ptr(out) if partition_size == 0 else None, _ptr(q), _dt(q),
                          _ptr(k_cache), _ptr(v_cache), _dt(k_cache), _ptr(k_scale), _ptr(v_scale),
                          _i32(block_tables, "block_tables"), block_tables.shape[1],
                          _i32(context_lens, "context_lens"), B, hq, hkv, d, bs, float(scale),
                          int(partition_size), int(max_partitions), _ptr(part_max),
                          _ptr(part_sum), _ptr(part_out), _stream(stream))
    _check("pa_decode", st)


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      partition_size, max_partitions, k_scale=None, v_scale=None, stream=None):
    """Split-K decode + reduce into out [B, Hq, D] with the partials in the
    library's static per-GPU scratch (no device memory from the caller)."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    B, hq = q.shape[0], q.shape[1]
    if q.shape[2] != d or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent decode shapes")
    if out is None or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    st = load().pa_decode_noalloc(_ptr(out), _ptr(q), _dt(q), _ptr(k_cache), _ptr(v_cache),
                                  _dt(k_cache), _ptr(k_scale), _ptr(v_scale),
                                  _i32(block_tables, "block_tables"), block_tables.shape[1],
                                  _i32(context_lens, "context_lens"), B, hq, hkv, d, bs,
                                  float(scale), int(partition_size), int(max_partitions),
                                  _stream(stream))
    _check("pa_decode_noalloc", st)


def pa_read_probe(buf, chunk_ids, sink, stream=None):
    """Read the 4 KB chunks of buf (a device tensor) in chunk_ids' order (a
    measurement aid: the decode's block-tile access pattern)."""
    nbytes = buf.numel() * buf.element_size()
    st = load().pa_read_probe(_ptr(buf), nbytes, _i32(chunk_ids, "chunk_ids"), chunk_ids.numel(),
                              _ptr(sink), sink.numel() * sink.element_size(), _stream(stream))
    _check("pa_read_probe", st)


def pa_decode_noalloc_max_bytes():
    return int(load().pa_decode_noalloc_max_bytes())


def pa_decode_append(out, q, k_new, v_new, new_slots, k_cache, v_cache, block_tables,
                     context_lens, scale, k_scale=None, v_scale=None, partition_size=0,
                     max_partitions=1, part_max=None, part_sum=None, part_out=None, plan=None,
                     stream=None):
    """pa_kv_append of each sequence's newest token (k_new, v_new [B, Hkv, D],
    new_slots int32 [B], -1 to skip; all three None: no append) and
    pa_decode, in one launch.  plan: a buffer pa_decode_plan filled for the
    same batch and arguments (skips the launch's prologue)."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    B, hq = q.shape[0], q.shape[1]
    if q.shape[2] != d or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent decode shapes")
    if (k_new is None) != (v_new is None) or (k_new is None) != (new_slots is None):
        raise ValueError("k_new, v_new and new_slots go together")
    if k_new is not None:
        if tuple(k_new.shape) != (B, hkv, d) or tuple(v_new.shape) != (B, hkv, d):
            raise ValueError("k_new/v_new must be [B, num_kv_heads, head_dim]")
        if k_new.dtype != q.dtype or v_new.dtype != q.dtype or new_slots.numel() != B:
            raise ValueError("k_new/v_new must have q's dtype; new_slots one entry per sequence")
    if partition_size > 0:
        want = (B, hq, max_partitions)
        for t in (part_max, part_sum):
            if t is None or tuple(t.shape) != want or t.dtype != torch.float32:
                raise ValueError("part_max/part_sum must be float32 %s" % (want,))
        if part_out is None or tuple(part_out.shape) != want + (d,):
            raise ValueError("part_out must be float32 %s" % (want + (d,),))
    elif out is None or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    st = load().pa_decode_append(_ptr(out) if partition_size == 0 else None, _ptr(q), _dt(q),
                                 _ptr(k_new), _ptr(v_new),
                                 None if new_slots is None else _i32(new_slots, "new_slots"),
                                 _ptr(k_cache), _ptr(v_cache), _dt(k_cache), _ptr(k_scale),
                                 _ptr(v_scale), _i32(block_tables, "block_tables"),
                                 block_tables.shape[1], _i32(context_lens, "context_lens"), B, hq,
                                 hkv, d, bs, float(scale), int(partition_size),
                                 int(max_partitions), _ptr(part_max), _ptr(part_sum),
                                 _ptr(part_out), _plan_ptr(plan), _plan_bytes(plan),
                                 _stream(stream))
    _check("pa_decode_append", st)


def pa_decode_cascade(q, k_cache, v_cache, block_tables, context_lens, scale, group_start,
                      group_seqs, group_prefix_lens, max_group_size, partition_size,
                      max_partitions, part_max, part_sum, part_out, k_scale=None, v_scale=None,
                      plan=None, k_new=None, v_new=None, new_slots=None, stream=None):
    """Split-K partials like pa_decode, reading each prefix group's shared
    partitions once for up to 16/G members at a time.  group_start int32
    [num_groups + 1], group_seqs int32 [members], group_prefix_lens int32
    [num_groups]."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    B, hq = q.shape[0], q.shape[1]
    if q.shape[2] != d or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("inconsistent decode shapes")
    if partition_size <= 0:
        raise ValueError("pa_decode_cascade needs partition_size > 0")
    want = (B, hq, max_partitions)
    for t in (part_max, part_sum):
        if t is None or tuple(t.shape) != want or t.dtype != torch.float32:
            raise ValueError("part_max/part_sum must be float32 %s" % (want,))
    if part_out is None or tuple(part_out.shape) != want + (d,):
        raise ValueError("part_out must be float32 %s" % (want + (d,),))
    ng = group_prefix_lens.numel()
    if group_start.numel() != ng + 1:
        raise ValueError("group_start must have num_groups + 1 entries")
    if (k_new is None) != (v_new is None) or (k_new is None) != (new_slots is None):
        raise ValueError("k_new, v_new and new_slots go together")
    if k_new is not None and (tuple(k_new.shape) != (B, hkv, d) or k_new.dtype != q.dtype
                              or tuple(v_new.shape) != (B, hkv, d) or new_slots.numel() != B):
        raise ValueError("k_new/v_new must be [B, num_kv_heads, head_dim] of q's dtype")
    st = load().pa_decode_cascade(_ptr(q), _dt(q), _ptr(k_new), _ptr(v_new),
                                  None if new_slots is None else _i32(new_slots, "new_slots"),
                                  _ptr(k_cache), _ptr(v_cache), _dt(k_cache),
                                  _ptr(k_scale), _ptr(v_scale), _i32(block_tables, "block_tables"),
                                  block_tables.shape[1], _i32(context_lens, "context_lens"), B,
                                  _i32(group_start, "group_start"), _i32(group_seqs, "group_seqs"),
                                  _i32(group_prefix_lens, "group_prefix_lens"), ng,
                                  int(max_group_size), hq, hkv, d, bs, float(scale),
                                  int(partition_size), int(max_partitions), _ptr(part_max),
                                  _ptr(part_sum), _ptr(part_out), _plan_ptr(plan),
                                  _plan_bytes(plan), _stream(stream))
    _check("pa_decode_cascade", st)


def pa_decode_multi(q, query_start_loc, max_query_len, k_cache, v_cache, block_tables,
                    context_lens, scale, partition_size, max_partitions, part_max, part_sum,
                    part_out, k_scale=None, v_scale=None, plan=None, k_new=None, v_new=None,
                    new_slots=None, stream=None):
    """Split-K partials for q_b causal query tokens per sequence: q [T, Hq, D]
    with T = query_start_loc[-1]; partials [T, Hq, max_partitions] (+ [D]).
    k_new, v_new [T, Hkv, D] and new_slots int32 [T] (-1 to skip): the query
    tokens' K/V, appended in the same launch (all three None: no append)."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    T, hq = q.shape[0], q.shape[1]
    B = context_lens.numel()
    if q.shape[2] != d or block_tables.shape[0] != B or query_start_loc.numel() != B + 1:
        raise ValueError("inconsistent multi-query decode shapes")
    if partition_size <= 0:
        raise ValueError("pa_decode_multi needs partition_size > 0")
    want = (T, hq, max_partitions)
    for t in (part_max, part_sum):
        if t is None or tuple(t.shape) != want or t.dtype != torch.float32:
            raise ValueError("part_max/part_sum must be float32 %s" % (want,))
    if part_out is None or tuple(part_out.shape) != want + (d,):
        raise ValueError("part_out must be float32 %s" % (want + (d,),))
    if (k_new is None) != (v_new is None) or (k_new is None) != (new_slots is None):
        raise ValueError("k_new, v_new and new_slots go together")
    if k_new is not None and (tuple(k_new.shape) != (T, hkv, d) or k_new.dtype != q.dtype
                              or tuple(v_new.shape) != (T, hkv, d) or v_new.dtype != q.dtype
                              or new_slots.numel() != T):
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim] of q's dtype and "
                         "new_slots one entry per query token")
    st = load().pa_decode_multi(_ptr(q), _dt(q), _ptr(k_new), _ptr(v_new),
                                None if new_slots is None else _i32(new_slots, "new_slots"),
                                _i32(query_start_loc, "query_start_loc"),
                                int(max_query_len), _ptr(k_cache), _ptr(v_cache), _dt(k_cache),
                                _ptr(k_scale), _ptr(v_scale), _i32(block_tables, "block_tables"),
                                block_tables.shape[1], _i32(context_lens, "context_lens"), B, hq,
                                hkv, d, bs, float(scale), int(partition_size), int(max_partitions),
                                _ptr(part_max), _ptr(part_sum), _ptr(part_out), _plan_ptr(plan),
                                _plan_bytes(plan), _stream(stream))
    _check("pa_decode_multi", st)


def pa_decode_splitk_reduce(out, part_max, part_sum, part_out, context_lens, partition_size,
                            stream=None):
    """Merge pa_decode's split-K partials into out [B, Hq, D]."""
    B, hq, pmax, d = part_out.shape
    if tuple(out.shape) != (B, hq, d):
        raise ValueError("out must be [B, Hq, D]")
    st = load().pa_decode_splitk_reduce(_ptr(out), _dt(out), _ptr(part_max), _ptr(part_sum),
                                        _ptr(part_out), _i32(context_lens, "context_lens"), B, hq,
                                        d, int(partition_size), pmax, _stream(stream))
    _check("pa_decode_splitk_reduce", st)


def pa_prefill_chunk(out, q, query_start_loc, max_query_len, k_cache, v_cache, block_tables,
                     context_lens, scale, k_scale=None, v_scale=None, stream=None):
    """out, q [total_q, Hq, D]; query_start_loc int32 [C+1]; block_tables [C, W]."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    total_q, hq = q.shape[0], q.shape[1]
    C = context_lens.numel()
    if query_start_loc.numel() != C + 1 or block_tables.shape[0] != C or q.shape[2] != d:
        raise ValueError("inconsistent prefill shapes")
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    st = load().pa_prefill_chunk(_ptr(out), _ptr(q), _dt(q), _i32(query_start_loc, "query_start_loc"),
                                 C, int(max_query_len), _ptr(k_cache), _ptr(v_cache), _dt(k_cache),
                                 _ptr(k_scale), _ptr(v_scale), _i32(block_tables, "block_tables"),
                                 block_tables.shape[1], _i32(context_lens, "context_lens"), hq, hkv,
                                 d, bs, float(scale), _stream(stream))
    _check("pa_prefill_chunk", st)
