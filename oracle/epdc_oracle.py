"""CPU oracle for MoE token dispatch and combine.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this directory.  The HIP library never calls it and
shares no code, table or constant generator with it.

Every function is the plain definition of one step, written with numpy in the
order the pages state it, with no blocking or fusion.  Hidden rows are handled
as raw bf16 bit patterns (``uint16``) so that copies are compared bit for bit.

Sources (page title, then the section the step follows):

* [axolotl] "integrations.expert_parallel.torch_dispatch" (axolotl API docs):
  module overview (DeepEP-compatible send layout, K-wide local ids and
  weights), ``compute_send_counts``, ``build_send_layout``, ``dispatch``,
  ``combine``, ``chunk_bounds``, ``dispatch_chunked_forward``.
* [uccl] "nemo_automodel.components.moe.uccl_ep.buffer" (NeMo AutoModel API
  docs): ``Buffer.get_dispatch_layout``, ``Buffer.dispatch`` (fp8 tuple with
  one float scale per 128 channels), ``Buffer.combine``,
  ``Buffer.low_latency_dispatch``.
* [vllm] "vllm.model_executor.layers.fused_moe.prepare_finalize" (vLLM API
  docs): ``BatchedPrepareAndFinalize.prepare`` / ``finalize``.
* [nemo] "nemo_automodel.components.moe.megatron.token_dispatcher" (NeMo
  AutoModel API docs): ``TokenDispatcherConfig.moe_router_dtype`` (fp32 for
  routing and for the weighted average of expert outputs).

Readings taken where the pages are silent (each is listed in the design
notes): combine is weighted per slot and accumulates in float32, product
rounded then sum rounded, k ascending, starting from +0.0, rounded once to
bf16 (nearest, ties to even); fp8 is OCP E4M3 (``float8_e4m3fn``) with
``scale = amax / 448`` in float32, the quotient ``x / scale`` rounded to
float32 and then to the nearest e4m3 value (ties to even), saturating at 448,
and an all-zero group giving scale 0 and code 0x00; a power-of-two scale is
the smallest power of two at or above amax / 448, its UE8M0 byte is the
exponent plus 127 (at least 0, i.e. 2^-127), and four such bytes pack into an
int32 with the lowest group in the lowest byte.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against brute force, closed forms, library routines (numpy sorts and
bincounts, torch's bf16 and float8_e4m3fn conversions) and a hand-worked
example; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "chunk_bounds",
    "validate_routing",
    "compute_send_counts",
    "build_send_layout",
    "dispatch_permute",
    "bf16_to_f32",
    "f32_to_bf16",
    "e4m3_decode",
    "e4m3_encode",
    "round_scale_pow2",
    "ue8m0_encode",
    "ue8m0_decode",
    "pack_ue8m0",
    "unpack_ue8m0",
    "quantize_rows_fp8",
    "dequantize_rows_fp8",
    "dispatch_permute_fp8",
    "batched_prepare",
    "batched_prepare_fp8",
    "scale_storage",
    "regroup_by_expert",
    "combine",
    "combine_partials",
    "FP8_MAX",
    "FP8_GROUP",
    "UE8M0_BIAS",
    "SCALE_FORMATS",
]

FP8_MAX = 448.0   # largest finite OCP E4M3 magnitude (S.1111.110)
FP8_GROUP = 128   # channels per fp32 scale ([uccl] Buffer.dispatch)
UE8M0_BIAS = 127  # UE8M0: 8 exponent bits, no sign, no mantissa
SCALE_FORMATS = ("f32", "pow2", "ue8m0")


# --------------------------------------------------------------------------
# Routing metadata
# --------------------------------------------------------------------------

def chunk_bounds(num_tokens: int, chunks: int):
    """[axolotl] chunk_bounds: ``chunks`` contiguous [start, end) ranges.

    All chunks but the last hold ``num_tokens // chunks`` tokens; the last one
    takes the remainder, so leading chunks are empty when num_tokens < chunks.
    """
    if chunks < 1:
        raise ValueError("chunks must be >= 1")
    size = num_tokens // chunks
    out = []
    for i in range(chunks):
        start = i * size
        end = num_tokens if i == chunks - 1 else (i + 1) * size
        out.append((start, end))
    return out


def validate_routing(topk_idx: np.ndarray, num_experts: int) -> None:
    """Preconditions of the routing input ([axolotl] dispatch; [uccl]
    Buffer.dispatch): int64 ids in [-1, E) with -1 meaning unrouted, and the
    routed ids of one token distinct (a router's top-k never repeats)."""
    idx = np.asarray(topk_idx)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [T, K]")
    if idx.size and (idx.min() < -1 or idx.max() >= num_experts):
        raise ValueError("expert id outside [-1, E)")
    for t in range(idx.shape[0]):
        routed = idx[t][idx[t] >= 0]
        if len(np.unique(routed)) != len(routed):
            raise ValueError(f"token {t} repeats an expert id")


def compute_send_counts(topk_idx, num_ranks, num_local_experts, num_chunks=1):
    """[axolotl] compute_send_counts and [uccl] Buffer.get_dispatch_layout.

    Returns ``dest`` int32 [T,K] (owning destination of each slot, -1 where
    unrouted), ``is_in_rank`` uint8 [T,P] (token has at least one expert on
    destination p), ``send_counts`` int32 [C,P] (tokens sent to p from chunk c)
    and ``tokens_per_expert`` int32 [C,E] (routed slots naming expert e in
    chunk c).  Destination p owns experts [p*E_local, (p+1)*E_local).
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    P, El = int(num_ranks), int(num_local_experts)
    E = P * El
    validate_routing(idx, E)

    dest = np.where(idx >= 0, idx // El, -1).astype(np.int32)
    is_in_rank = np.zeros((T, P), dtype=np.uint8)
    for p in range(P):
        is_in_rank[:, p] = (dest == p).any(axis=1)

    C = int(num_chunks)
    send_counts = np.zeros((C, P), dtype=np.int32)
    tokens_per_expert = np.zeros((C, E), dtype=np.int32)
    for c, (s, e) in enumerate(chunk_bounds(T, C)):
        send_counts[c] = is_in_rank[s:e].sum(axis=0)
        for ex in range(E):
            tokens_per_expert[c, ex] = int((idx[s:e] == ex).sum())
    return dest, is_in_rank, send_counts, tokens_per_expert


def build_send_layout(topk_idx, topk_weights, num_ranks, num_local_experts):
    """[axolotl] build_send_layout plus the module overview's layout contract.

    Send rows are ordered destination-major, then token-ascending: for p in
    0..P-1 and, inside p, for every token t with is_in_rank[t,p] in ascending
    order, the next row n is taken.  Row n carries
    ``send_token_idx[n] = t``, ``send_rank[n] = p``,
    ``send_idx[n,k] = id - p*E_local`` on slots owned by p and -1 elsewhere,
    ``send_w[n,k] = w[t,k]`` on those slots and +0.0 elsewhere.
    ``token_row[t,k]`` is the send row of slot k's owner (-1 if unrouted); it
    is the inverse map that combine uses to find the expert output of a slot.
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float32)
    T, K = idx.shape
    P, El = int(num_ranks), int(num_local_experts)
    dest, is_in_rank, _, _ = compute_send_counts(idx, P, El, 1)

    N = int(is_in_rank.sum())
    send_token_idx = np.zeros(N, dtype=np.int32)
    send_rank = np.zeros(N, dtype=np.int32)
    send_idx = np.full((N, K), -1, dtype=np.int32)
    send_w = np.zeros((N, K), dtype=np.float32)
    token_row = np.full((T, K), -1, dtype=np.int32)

    n = 0
    for p in range(P):
        for t in np.flatnonzero(is_in_rank[:, p]):
            owned = dest[t] == p
            send_token_idx[n] = t
            send_rank[n] = p
            send_idx[n, owned] = idx[t, owned] - p * El
            send_w[n, owned] = w[t, owned]
            token_row[t, owned] = n
            n += 1
    assert n == N
    return send_token_idx, send_rank, send_idx, send_w, token_row


def dispatch_permute(x_bits, send_token_idx):
    """[axolotl] dispatch: row n of the send buffer is hidden row
    send_token_idx[n], copied bit for bit (tokens with no routed expert are
    not sent)."""
    x = np.asarray(x_bits)
    return x[np.asarray(send_token_idx, dtype=np.int64)].copy()


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_to_f32(bits):
    """bf16 is the upper half of an IEEE binary32 word."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_bf16(values):
    """Round float32 to bf16, to nearest with ties to even.

    bf16 keeps the upper 16 bits of binary32.  The two candidates are the
    truncated magnitude and the next bf16 magnitude up; the dropped 16 bits
    decide, and an exact half picks the candidate whose last kept bit is 0
    (past the largest bf16 the next magnitude up is infinity).  The pages
    leave NaN open; reading: a NaN stays a quiet NaN, its sign and payload
    unspecified (those of a NaN produced by arithmetic differ from one
    machine to another, so comparisons take any two NaNs as equal); this
    function writes the canonical 0x7FC0.
    """
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    lower = u & np.uint32(0xFFFF0000)
    upper = lower + np.uint32(0x10000)
    rem = u & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    lower_even = ((lower >> np.uint32(16)) & np.uint32(1)) == 0
    pick_upper = (rem > half) | ((rem == half) & ~lower_even)
    out = np.where(pick_upper, upper, lower)
    out = (out >> np.uint32(16)).astype(np.uint16)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    return np.where(is_nan, np.uint16(0x7FC0), out).astype(np.uint16)


def e4m3_decode(codes):
    """Value of OCP E4M3 (float8_e4m3fn) codes: 1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); no
    infinities; S.1111.111 is NaN.  Returned as float64 (exact)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# Positive finite e4m3 values in code order 0x00..0x7E (ascending magnitude).
_E4M3_POS = e4m3_decode(np.arange(0x7F))


def e4m3_encode(values):
    """Nearest OCP E4M3 code of each float32 value, ties to the even code
    (mantissa LSB 0); magnitudes at or above 448, infinities included,
    saturate to 448; the sign bit is kept, so -0.0 and negative values that
    round to zero give 0x80.  Any NaN gives the NaN code 0x7F."""
    v = np.asarray(values, dtype=np.float32)
    sign = (v.view(np.uint32) >> np.uint32(31)).astype(np.int64)
    with np.errstate(invalid="ignore"):        # a signalling NaN quietens
        mag = np.abs(v.astype(np.float64))
    hi = np.searchsorted(_E4M3_POS, mag, side="left")        # POS[hi] >= mag
    hi = np.clip(hi, 0, len(_E4M3_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_E4M3_POS) - 1)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(mag >= FP8_MAX, 0x7E, code)
    code = np.where(mag == 0.0, 0, code)
    code = code | (sign << 7)
    return np.where(np.isnan(mag), 0x7F, code).astype(np.uint8)


def round_scale_pow2(s):
    """[uccl] Buffer.low_latency_dispatch ``round_scale``: the scale becomes a
    power of two.  Reading: the smallest power of two that is >= s, so that
    x / scale still lies within the e4m3 range; 0 stays 0, and an infinite
    scale (a group holding an infinity) stays infinite.  Input and output
    float32 (every such power of two from 2^-149 up is a float32)."""
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    fin = np.isfinite(s64)
    m, e = np.frexp(np.where(fin, s64, 1.0))     # s = m * 2^e with 0.5 <= m < 1
    p = np.where(m == 0.5, s64, np.ldexp(1.0, e))
    p = np.where(fin, p, s64)
    return np.where(s64 == 0.0, 0.0, p).astype(np.float32)


def ue8m0_encode(p):
    """UE8M0 byte of a power of two p ([uccl] Buffer.low_latency_dispatch
    ``use_ue8m0``): 8 exponent bits with bias 127, no sign and no mantissa,
    so 2^e is stored as e + 127.  Powers below 2^-127, and 0, take the
    smallest code 0x00 (2^-127): a larger scale than asked for, which keeps
    x / scale in range.  The largest scale a finite bf16 group can ask for
    is 2^120 (code 247), so no finite group reaches the top codes; an
    infinite scale takes 0xFF, the code past every power (its value taken
    as infinity, so the group's finite elements quantize to zero)."""
    p64 = np.asarray(p, dtype=np.float32).astype(np.float64)
    e = np.frexp(np.where(np.isfinite(p64), p64, 1.0))[1] - 1      # p = 2^e
    b = np.where(p64 > 0, np.clip(e + UE8M0_BIAS, 0, 254), 0)
    b = np.where(np.isinf(p64), 255, b)
    return b.astype(np.uint8)


def ue8m0_decode(b):
    """float32 value 2^(b - 127) of UE8M0 bytes 0..254; 255 (2^128) is past
    float32 and decodes to infinity."""
    b = np.asarray(b, dtype=np.int64)
    with np.errstate(over="ignore"):
        return np.ldexp(1.0, b - UE8M0_BIAS).astype(np.float32)


def pack_ue8m0(b):
    """[uccl] Buffer.low_latency_dispatch: UE8M0 scales packed four to a
    32-bit int ([.., H/512] int).  Reading: int j holds the bytes of groups
    4j..4j+3 with group 4j in the least significant byte."""
    b = np.asarray(b, dtype=np.uint8).astype(np.uint32)
    *lead, G = b.shape
    if G % 4:
        raise ValueError("UE8M0 packing needs a multiple of 4 groups (H % 512 == 0)")
    b = b.reshape(*lead, G // 4, 4)
    word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    return word.astype(np.uint32).view(np.int32)


def unpack_ue8m0(packed):
    """Inverse of pack_ue8m0: the group bytes, [.., 4 * words] uint8."""
    w = np.asarray(packed, dtype=np.int32).view(np.uint32)
    parts = [(w >> np.uint32(8 * i)) & np.uint32(0xFF) for i in range(4)]
    return np.stack(parts, axis=-1).reshape(*w.shape[:-1], -1).astype(np.uint8)


def quantize_rows_fp8(x_bits, scale_fmt="f32"):
    """[uccl] Buffer.dispatch / low_latency_dispatch fp8 input: e4m3 rows plus
    one scale per token per 128 channels.

    For each group of 128 channels: amax = max |x| (exact) and s =
    fl32(amax / 448).  The scale is s (``f32``), the smallest power of two
    >= s (``pow2``, [uccl] ``round_scale``), or that power as a UE8M0 byte
    (``ue8m0``, [uccl] ``use_ue8m0``; the quantizer then divides by the
    byte's value 2^(b-127)).  q = e4m3(fl32(x / scale)).  A group whose amax
    is 0 gets all codes 0x00 and scale 0.0 (byte 0x00 in ``ue8m0``).  The
    pages leave non-finite inputs open; reading: NaN elements do not count
    toward amax (as a running fmax) and always encode to the NaN code 0x7F
    (also in a group with no other non-zero element), and a group holding
    an infinity gets an infinite scale, so its finite elements give zeros.
    Returns (uint8 [R,H], scales): float32 [R, H/128] for ``f32`` and
    ``pow2``, int32 [R, H/512] (pack_ue8m0) for ``ue8m0``.
    """
    if scale_fmt not in SCALE_FORMATS:
        raise ValueError(f"scale_fmt must be one of {SCALE_FORMATS}")
    x = bf16_to_f32(x_bits)
    R, H = x.shape
    if H % FP8_GROUP:
        raise ValueError("H must be a multiple of 128 for fp8")
    g = x.reshape(R, H // FP8_GROUP, FP8_GROUP)
    amax = np.where(np.isnan(g), np.float32(0.0), np.abs(g)).max(axis=2)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    if scale_fmt == "pow2":
        scale = round_scale_pow2(scale)
    elif scale_fmt == "ue8m0":
        byte = ue8m0_encode(round_scale_pow2(scale))
        scale = np.where(amax > 0, ue8m0_decode(byte), np.float32(0.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    with np.errstate(invalid="ignore"):           # inf / inf: NaN, encoded as such
        quot = (g / safe[:, :, None]).astype(np.float32)
    q = e4m3_encode(quot)
    zero_group = np.where(np.isnan(g), np.uint8(0x7F), np.uint8(0))
    q = np.where((scale > 0)[:, :, None], q, zero_group)
    q = q.reshape(R, H).astype(np.uint8)
    if scale_fmt == "ue8m0":
        return q, pack_ue8m0(byte)
    return q, scale


def dequantize_rows_fp8(q, scales):
    """bf16 bits of fl32(decode(q) * scale) per element: the expert output of
    an identity expert fed with the fp8 rows (used as the combine input)."""
    q = np.asarray(q, dtype=np.uint8)
    R, H = q.shape
    vals = e4m3_decode(q).astype(np.float32).reshape(R, H // FP8_GROUP, FP8_GROUP)
    prod = (vals * np.asarray(scales, dtype=np.float32)[:, :, None]).astype(np.float32)
    return f32_to_bf16(prod.reshape(R, H))


def dispatch_permute_fp8(x_bits, send_token_idx):
    """fp8 quantize-on-dispatch: row n holds the quantized hidden row of token
    send_token_idx[n] and its scales (quantization is per token, so it does
    not depend on which destination the row goes to)."""
    q, s = quantize_rows_fp8(x_bits)
    rows = np.asarray(send_token_idx, dtype=np.int64)
    return q[rows].copy(), s[rows].copy()


# --------------------------------------------------------------------------
# Expert-batched layout
# --------------------------------------------------------------------------

def batched_prepare(x_bits, topk_idx, first_expert, num_local_experts,
                    max_num_tokens):
    """[vllm] BatchedPrepareAndFinalize.prepare, unquantized branch.

    The buffer [E_local, max_num_tokens, H] starts zeroed.  For local expert e
    (global id first+e) the tokens that name it in any slot take slots
    0, 1, 2, ... in ascending token order (running count minus one), and the
    token's hidden row is stored there.  tokens_per_expert[e] is that count.
    token_row[t,k] = e*max_num_tokens + slot for local slots, else -1.
    """
    x = np.asarray(x_bits, dtype=np.uint16)
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    H = x.shape[1]
    El, M = int(num_local_experts), int(max_num_tokens)
    b_x = np.zeros((El, M, H), dtype=np.uint16)
    tokens_per_expert = np.zeros(El, dtype=np.int32)
    token_row = np.full((T, K), -1, dtype=np.int32)
    for e in range(El):
        hit_slots = idx == (first_expert + e)
        tokens = np.flatnonzero(hit_slots.any(axis=1))
        if len(tokens) > M:
            raise ValueError(f"expert {first_expert + e} receives {len(tokens)}"
                             f" tokens > max_num_tokens={M}")
        tokens_per_expert[e] = len(tokens)
        for slot, t in enumerate(tokens):
            b_x[e, slot] = x[t]
            token_row[t, hit_slots[t]] = e * M + slot
    return b_x, tokens_per_expert, token_row


def batched_prepare_fp8(x_bits, topk_idx, first_expert, num_local_experts,
                        max_num_tokens, scale_fmt="f32"):
    """[uccl] Buffer.low_latency_dispatch with ``use_fp8`` (the received
    tokens per local expert as e4m3 rows [E_local, max, H] plus scales
    [E_local, max, H/128] float, or packed UE8M0 [E_local, max, H/512] int),
    and [vllm] BatchedPrepareAndFinalize.prepare, quantized branch (zeroed
    buffers, each expert's rows quantized per token).

    Quantization is per token and per 128 channels, so the buffer is the
    expert-batched gather of quantize_rows_fp8(x): slot s of expert e holds
    the codes and scales of the token batched_prepare puts there.  Padding
    slots hold codes 0x00 and scale 0 (int 0 in ``ue8m0``).  Returns
    (b_q uint8 [E_local, max, H], b_scale [E_local, max, H/128] float32 or
    [E_local, max, H/512] int32, tokens_per_expert, token_row); the scale
    array is in logical (expert, slot, group) order (scale_storage gives the
    memory order).
    """
    x = np.asarray(x_bits, dtype=np.uint16)
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    H = x.shape[1]
    El, M = int(num_local_experts), int(max_num_tokens)
    q, sc = quantize_rows_fp8(x, scale_fmt)
    _, tokens_per_expert, token_row = batched_prepare(x, idx, first_expert, El, M)
    b_q = np.zeros((El, M, H), dtype=np.uint8)
    b_scale = np.zeros((El, M, sc.shape[1]), dtype=sc.dtype)
    for e in range(El):
        tokens = np.flatnonzero((idx == (first_expert + e)).any(axis=1))
        for slot, t in enumerate(tokens):
            b_q[e, slot] = q[t]
            b_scale[e, slot] = sc[t]
    return b_q, b_scale, tokens_per_expert, token_row


def scale_storage(b_scale, col_major):
    """Memory order of an expert-batched scale array [E_local, max, G]:
    row-major, or ([uccl] Buffer.low_latency_dispatch) column-major in the
    last two dimensions, i.e. each expert's [max, G] block stored as [G, max].
    Returns the flat array in memory order."""
    b = np.asarray(b_scale)
    if col_major:
        b = b.transpose(0, 2, 1)
    return np.ascontiguousarray(b).reshape(-1)


# --------------------------------------------------------------------------
# Receive side: rows regrouped by local expert
# --------------------------------------------------------------------------

def regroup_by_expert(x_bits, recv_idx, recv_w, num_local_experts, align=1,
                      row_group=None, num_groups=1):
    """[nemo] MoEFlexTokenDispatcher.dispatch_postprocess and
    _DeepepManager.get_permuted_hidden_states_by_experts (the received rows
    permuted so that each local expert's rows are contiguous, with the
    number of tokens per expert); [nemo] TokenDispatcherConfig
    moe_router_expert_pad_multiple and [uccl] Buffer.dispatch
    expert_alignment (each expert's row count padded to a multiple).

    For local expert e = 0..E_local-1 in order, each received row r whose
    recv_idx names e (in ascending r) takes the next row of e's segment,
    which is then padded with zero rows to a multiple of ``align``.
    Returns perm_x [M,H] bf16 bits, perm_src [M] (the received row, -1 on
    padding), perm_w [M] (that slot's weight, 0 on padding),
    tokens_per_expert [E_local] (without padding), offsets [E_local+1]
    (padded segment starts; offsets[E_local] = M) and row_map [R,K] (the
    permuted row of slot k, -1 where the slot names no local expert).

    With ``row_group`` the rows are ``num_groups`` receive buffers laid end to
    end (on one GPU: the destination segments of a send buffer) and the bins
    are (group g, expert e) in g-major order, each regrouped as above; the
    counts and offsets then have num_groups*E_local (+1) entries.
    """
    x = np.asarray(x_bits, dtype=np.uint16)
    idx = np.asarray(recv_idx, dtype=np.int64)
    w = np.asarray(recv_w, dtype=np.float32)
    R, K = idx.shape
    H = x.shape[1]
    El, A = int(num_local_experts), int(align)
    if A < 1:
        raise ValueError("align must be >= 1")
    validate_routing(idx, El)
    G = int(num_groups)
    grp = np.zeros(R, dtype=np.int64) if row_group is None else np.asarray(row_group)
    if row_group is None and G != 1:
        raise ValueError("num_groups > 1 needs row_group")
    if R and (grp.min() < 0 or grp.max() >= G):
        raise ValueError("row_group outside [0, num_groups)")
    B = G * El
    counts = np.zeros(B, dtype=np.int32)
    members = []
    for b in range(B):
        g, e = divmod(b, El)
        rows = [r for r in range(R) if grp[r] == g and (idx[r] == e).any()]
        members.append(rows)
        counts[b] = len(rows)
    padded = [-(-int(c) // A) * A for c in counts]
    offsets = np.zeros(B + 1, dtype=np.int32)
    for b in range(B):
        offsets[b + 1] = offsets[b] + padded[b]
    M = int(offsets[B])
    perm_x = np.zeros((M, H), dtype=np.uint16)
    perm_src = np.full(M, -1, dtype=np.int32)
    perm_w = np.zeros(M, dtype=np.float32)
    row_map = np.full((R, K), -1, dtype=np.int32)
    for b in range(B):
        e = b % El
        for s, r in enumerate(members[b]):
            n = offsets[b] + s
            k = int(np.flatnonzero(idx[r] == e)[0])
            perm_x[n] = x[r]
            perm_src[n] = r
            perm_w[n] = w[r, k]
            row_map[r, k] = n
    return perm_x, perm_src, perm_w, counts, offsets, row_map


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------

def _add_biases(acc, biases):
    """[uccl] Buffer.combine ``bias``: one [T,H] tensor or a pair, added to
    the reduced tokens.  Reading: each bias (bf16) is added to the float32
    sum after the expert terms, in the order given, before the one rounding
    to bf16."""
    for b in biases:
        acc = (acc + bf16_to_f32(np.asarray(b, dtype=np.uint16))).astype(np.float32)
    return acc


def combine(y_bits, token_row, topk_weights, biases=()):
    """[axolotl] combine, [uccl] Buffer.combine / low_latency_combine,
    [vllm] BatchedPrepareAndFinalize.finalize: the weighted per-token sum of
    expert outputs back onto the source tokens.

    out[t] = bf16( sum over k = 0..K-1 with r = token_row[t,k] >= 0 of
    w[t,k] * y[r] ), accumulated in float32 ([nemo] moe_router_dtype): each
    product is rounded to float32, then added to the running float32 sum
    (which starts at +0.0) in ascending k.  Tokens with no routed slot give 0
    (plus the biases, if any).
    """
    y = np.asarray(y_bits, dtype=np.uint16)
    row = np.asarray(token_row, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float32)
    T, K = row.shape
    H = y.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)
    for k in range(K):
        r = row[:, k]
        m = r >= 0
        if not m.any():
            continue
        prod = (w[m, k][:, None] * bf16_to_f32(y[r[m]])).astype(np.float32)
        acc[m] = (acc[m] + prod).astype(np.float32)
    return f32_to_bf16(_add_biases(acc, biases))


def combine_partials(y_bits, token_row, biases=()):
    """[axolotl] module overview and combine: the local expert kernel already
    weights and sums over its slots, and combine sums the per-destination
    partial outputs back onto the source tokens, without weights ([uccl]
    Buffer.combine, when no topk_weights are given, adds the rows as they
    are).

    Each distinct row of token t (the send row of one destination; slots
    owned by the same destination share it) is added once, in the order of
    its first slot (k ascending), to a float32 sum that starts at +0.0; then
    the biases; then one rounding to bf16.
    """
    y = np.asarray(y_bits, dtype=np.uint16)
    row = np.asarray(token_row, dtype=np.int64)
    T, K = row.shape
    H = y.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)
    for t in range(T):
        seen = []
        for k in range(K):
            r = int(row[t, k])
            if r < 0 or r in seen:
                continue
            seen.append(r)
            acc[t] = (acc[t] + bf16_to_f32(y[r])).astype(np.float32)
    return f32_to_bf16(_add_biases(acc, biases))
