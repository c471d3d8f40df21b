"""Exact CPU definition of the paged lightning indexer (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module.  It is written from the pages' statement of the problem, in fp64
(or exact integers) wherever floating point is free to choose, and it shares
nothing with the HIP kernels.

Notation (fixed by the workload, not by the pages): H = 64 indexer heads,
D = 128 head dimension, 64 tokens per cache block.

Readings of the pages that this module takes (each one listed again in the
design notes of the repository):
  * the indexer score of query row r against key s is
        L[r, s] = k_scale[s] * sum_h w[r, h] * max(q[r, h, :] . k[s, :], 0)
    over the fp8-decoded values of q and k; the pages name this op
    ("fp8_paged_mqa_logits", vLLM PR #36250, Purpose) but do not print the
    formula, so the DeepSeek-V3.2 lightning-indexer definition is used;
  * the per-token query scale is folded into the head weights
    (w_eff = fl32(w * q_scale)), because ReLU is positively homogeneous;
  * row j of a request with context c and next_n query tokens sees
    limit = c - next_n + j + 1 keys; all later columns are -inf (clean logits,
    vLLM PR #36250 review thread);
  * top-k order is ascending column index, ties go to the lower index, rows
    with fewer than k visible keys return all of them then -1 padding;
  * -0.0 and +0.0 compare equal.
"""
import numpy as np

BLOCK = 64           # tokens per paged block
HEADS = 64           # indexer heads
DIM = 128            # indexer head dimension
VALUE_BYTES = BLOCK * DIM               # 8192 fp8 codes per block
BLOCK_BYTES = VALUE_BYTES + BLOCK * 4   # + 64 fp32 scales = 8448 bytes
FLT_MIN = np.float32(1.1754944e-38)
INV_448 = np.float32(1.0 / 448.0)       # fl32(1/448), as the quantiser multiplies by it


# --------------------------------------------------------------------------
# fp8 e4m3fn
# --------------------------------------------------------------------------
def e4m3fn_table():
    """Value of every fp8 e4m3fn code, from the bit definition, in float64.

    The cache stores torch.float8_e4m3fn values (vLLM PR #25869, review of
    cp_gather_indexer_k_quant_cache: ``.view(torch.float8_e4m3fn)``).  Sign bit 7,
    exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 is
    subnormal (m * 2^-9); exponent 15 with mantissa 7 is NaN; no infinities,
    so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3fn_table()
_POS = _TABLE[:127]          # codes 0x00..0x7E: the non-negative finite values, ascending


def fp8_encode(y):
    """Round float32 values to the nearest e4m3fn code, ties to the even code,
    saturating at +-448 (the finite maximum; the format has no infinity).

    Rounding is round-to-nearest-even: the pages quantise with a plain cast to
    the fp8 type after dividing by the scale (prhub summary of vLLM PR #47090,
    key source excerpt), which rounds to nearest even.  The magnitude is
    clamped to 448 first, so values just above 448 from rounding of the scale
    saturate instead of becoming NaN.  The sign bit of the input is kept, so
    -0.0 and negative values that round to zero give code 0x80.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 448.0)
    hi = np.searchsorted(_POS, a, side="left")        # _POS[hi] >= a
    hi = np.clip(hi, 0, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    mag = np.where(take_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def quantize_rows(x):
    """Dynamic per-row fp8 quantisation of float32 rows.

    Follows the tile quantiser of the prhub summary of vLLM PR #47090 (key
    source excerpt of ``_fused_norm_rope_kernel``): amax = max |x|;
    scale = max(amax * fl32(1/448), 1.1754944e-38); code = fp8(x / scale).
    All arithmetic is float32, as in that kernel: the scale is a float32
    product and the division is IEEE float32 division.  Returns
    (codes uint8 [N, L], scale float32 [N]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.maximum(amax * INV_448, FLT_MIN).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    return fp8_encode(y), scale


def quantize_q(q, w):
    """Query producer: one fp8 scale per query token over all H x D values,
    folded into that token's head weights.

    q: float32 [T, H, D] (bf16-representable), w: float32 [T, H].
    Returns (q_codes uint8 [T, H, D], w_eff float32 [T, H], q_scale float32 [T]).
    The quantiser is ``quantize_rows`` on the flattened token; the fold is
    w_eff = fl32(w * q_scale), valid because w*ReLU(s*x) = (w*s)*ReLU(x) for s > 0.
    """
    q = np.asarray(q, dtype=np.float32)
    T = q.shape[0]
    codes, scale = quantize_rows(q.reshape(T, -1))
    w_eff = (np.asarray(w, dtype=np.float32) * scale[:, None]).astype(np.float32)
    return codes.reshape(q.shape), w_eff, scale


# --------------------------------------------------------------------------
# rotary position embedding (fused producers)
# --------------------------------------------------------------------------
def rope_rotate(x, positions, cos_table, sin_table, rope_dim):
    """Rotate the first ``rope_dim`` values of every row of x by its token's
    position, in float32.

    The pages show the rotated pair being stored as ``r1`` at position 2i and
    ``r2`` at position 2i + 1 (prhub summary of vLLM PR #47090, key source
    excerpt of ``_fused_norm_rope_kernel``, MLA_CACHE_DS_MLA branch); they do
    not print the rotation or its tables.  Reading taken: pair i of a row is
    (x[2i], x[2i+1]) for 2i + 1 < rope_dim, the angle's cosine and sine are
    row ``positions[t]`` of the caller's tables (column i), and
        r1 = fl32(fl32(x1 * cos) - fl32(x2 * sin))
        r2 = fl32(fl32(x2 * cos) + fl32(x1 * sin))
    with every product and sum rounded to float32 on its own (no fused
    multiply-add).  Values at or past rope_dim are unchanged.

    x: float32 [T, ..., L] (the rotation acts on the last axis of every
    row); positions: int [T]; cos_table, sin_table: float32 [P, rope_dim/2].
    Returns float32 of x's shape.  The caller checks 0 <= positions < P.
    """
    x = np.array(x, dtype=np.float32, copy=True)
    half = rope_dim // 2
    if half == 0:
        return x
    pos = np.asarray(positions, dtype=np.int64)
    c = np.asarray(cos_table, dtype=np.float32)[pos, :half]     # [T, half]
    sn = np.asarray(sin_table, dtype=np.float32)[pos, :half]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c, sn = c.reshape(shape), sn.reshape(shape)
    x1 = x[..., 0:2 * half:2].copy()
    x2 = x[..., 1:2 * half:2].copy()
    x[..., 0:2 * half:2] = (x1 * c).astype(np.float32) - (x2 * sn).astype(np.float32)
    x[..., 1:2 * half:2] = (x2 * c).astype(np.float32) + (x1 * sn).astype(np.float32)
    return x


def quantize_q_rope(q, positions, cos_table, sin_table, rope_dim, w):
    """Fused query producer: rotate the first rope_dim values of every head
    of every query token (``rope_rotate``), then ``quantize_q``.

    A token whose position is outside [0, P) gets NaN codes (0x7F), a NaN
    scale and NaN folded weights (the library's signal for a caller error).
    Returns (q_codes uint8 [T, H, D], w_eff float32 [T, H], q_scale float32 [T]).
    """
    q = np.asarray(q, dtype=np.float32)
    pos = np.asarray(positions, dtype=np.int64)
    P = np.asarray(cos_table).shape[0]
    ok = (pos >= 0) & (pos < P)
    rot = q.copy()
    if ok.any():
        rot[ok] = rope_rotate(q[ok], pos[ok], cos_table, sin_table, rope_dim)
    codes, w_eff, scale = quantize_q(rot, w)
    codes[~ok] = 0x7F
    w_eff[~ok] = np.nan
    scale[~ok] = np.nan
    return codes, w_eff, scale


def k_rope_cache_write(k, positions, cos_table, sin_table, rope_dim, slot_mapping, cache):
    """Fused K producer: rotate the first rope_dim values of every K row
    (``rope_rotate``), quantise it and store it in the paged indexer cache
    (``k_cache_write``), in place.  A negative slot is skipped; a token whose
    position is outside [0, P) is stored as NaN codes (0x7F) and a NaN scale.
    """
    k = np.asarray(k, dtype=np.float32)
    pos = np.asarray(positions, dtype=np.int64)
    P = np.asarray(cos_table).shape[0]
    ok = (pos >= 0) & (pos < P)
    rot = k.copy()
    if ok.any():
        rot[ok] = rope_rotate(k[ok], pos[ok], cos_table, sin_table, rope_dim)
    k_cache_write(rot, slot_mapping, cache)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    bad = (~ok) & (slots >= 0)
    if bad.any():
        blk, off = slots[bad] // BLOCK, slots[bad] % BLOCK
        values = cache[:, :VALUE_BYTES].reshape(-1, BLOCK, DIM)
        scales = cache[:, VALUE_BYTES:BLOCK_BYTES].view(np.float32)
        values[blk, off] = 0x7F
        scales[blk, off] = np.nan
    return cache


# --------------------------------------------------------------------------
# paged cache
# --------------------------------------------------------------------------
def _block_values(cache, blk):
    return cache[blk, :VALUE_BYTES].reshape(BLOCK, DIM)


def _block_scales(cache, blk):
    return cache[blk, VALUE_BYTES:BLOCK_BYTES].copy().view(np.float32)


def k_cache_write(k, slot_mapping, cache):
    """Quantise K rows and store them in the paged indexer cache, in place.

    Layout of one block (vLLM PR #25869, review of
    cp_gather_indexer_k_quant_cache): ``block_size * head_dim`` fp8 values,
    token t at bytes [t*D, (t+1)*D), then ``block_size`` fp32 scales, token t
    at byte ``block_size*D + 4t``.  Slot s lives in block s // 64 at offset
    s % 64; a negative slot is skipped.
    k: float32 [N, D] (bf16-representable); slot_mapping: int [N];
    cache: uint8 [num_blocks, BLOCK_BYTES] (modified).
    """
    codes, scale = quantize_rows(k)
    slot_mapping = np.asarray(slot_mapping, dtype=np.int64)
    keep = slot_mapping >= 0
    blk, off = slot_mapping[keep] // BLOCK, slot_mapping[keep] % BLOCK
    values = cache[:, :VALUE_BYTES].reshape(-1, BLOCK, DIM)      # views into the cache
    scales = cache[:, VALUE_BYTES:BLOCK_BYTES].view(np.float32)  # [num_blocks, 64]
    values[blk, off] = codes[keep]
    scales[blk, off] = scale[keep]
    return cache


def gather_indexer_k(cache, block_table, cu_seq_lens, total_tokens):
    """Paged -> contiguous copy of each request's fp8 K and fp32 scales.

    Follows the preallocated rewrite in the review of
    cp_gather_indexer_k_quant_cache (vLLM PR #25869): request b owns rows
    [cu[b], cu[b+1]); an empty request is skipped; its full blocks are copied
    whole; the last block contributes only the first ``remaining`` tokens of
    values and scales.  Rows not owned by any request stay zero.
    Returns (values uint8 [total, D], scales float32 [total]).
    """
    dst_v = np.zeros((total_tokens, DIM), dtype=np.uint8)
    dst_s = np.zeros((total_tokens,), dtype=np.float32)
    cu = np.asarray(cu_seq_lens).tolist()
    for b in range(len(cu) - 1):
        s = cu[b + 1] - cu[b]
        if s <= 0:
            continue
        start = cu[b]
        nblk = -(-s // BLOCK)
        blocks = np.asarray(block_table[b][:nblk]).tolist()
        full = s // BLOCK
        for i in range(full):
            rows = slice(start + i * BLOCK, start + (i + 1) * BLOCK)
            dst_v[rows] = _block_values(cache, blocks[i])
            dst_s[rows] = _block_scales(cache, blocks[i])
        rem = s - full * BLOCK
        if rem > 0:
            rows = slice(start + full * BLOCK, start + full * BLOCK + rem)
            dst_v[rows] = _block_values(cache, blocks[-1])[:rem]
            dst_s[rows] = _block_scales(cache, blocks[-1])[:rem]
    return dst_v, dst_s


# --------------------------------------------------------------------------
# logits
# --------------------------------------------------------------------------
def decode_limits(context_lens, next_n):
    """Causal limit (number of visible keys) of every decode row, and its request.

    Row r = b*next_n + j is query token j of request b; the request's context
    length c counts its own new tokens, so token j sees keys [0, c - next_n + j + 1).
    """
    lim, req = [], []
    for b, c in enumerate(np.asarray(context_lens).tolist()):
        for j in range(next_n):
            lim.append(c - next_n + j + 1)
            req.append(b)
    return np.asarray(lim, dtype=np.int64), np.asarray(req, dtype=np.int64)


def _score(q_codes_row, w_row, k_codes, k_scale):
    """Indexer score of one query row [H, D] against keys [S, D], in float64.

    The fp8 values times 2^9 are integers below 2^18, so each head's dot
    product is an integer below 2^43 and the float64 matrix product computes
    it exactly in any order; the head sum runs h = 0..63 in float64.
    """
    qi = _TABLE[q_codes_row] * 512.0          # [H, D] exact integers
    ki = _TABLE[k_codes] * 512.0              # [S, D] exact integers
    d = (qi @ ki.T) * 2.0 ** -18              # [H, S] exact
    acc = np.zeros(k_codes.shape[0], dtype=np.float64)
    for h in range(HEADS):
        acc += np.float64(w_row[h]) * np.maximum(d[h], 0.0)
    return np.asarray(k_scale, dtype=np.float64) * acc


def paged_mqa_logits(q_codes, w, cache, block_table, context_lens, next_n, width,
                     rows=None, clean=True):
    """FP8 paged MQA logits with the causal -inf mask (clean logits).

    vLLM PR #36250 (Purpose): ``fp8_paged_mqa_logits`` scores every query
    token of every request against that request's paged K, one context length
    per request.  Keys are addressed through the block table exactly as the
    cache layout of vLLM PR #25869 (review of cp_gather_indexer_k_quant_cache)
    stores them.  Columns at or beyond a row's limit, up to ``width``, are -inf
    (the review thread's "clean logits").  Dequantisation is float64 here (the
    review thread insists on fp32, never fp16).

    q_codes: uint8 [B, next_n, H, D]; w: float32 [B*next_n, H];
    cache: uint8 [num_blocks, BLOCK_BYTES]; block_table: int [B, max_blocks];
    context_lens: int [B].  ``rows`` optionally restricts the computation to
    a subset of row ids (other rows are left NaN).  ``clean=False`` is the
    review's non-clean variant: columns from the end of the request's last
    key block on are not written (NaN here, untouched on the GPU).
    Returns float64 [B*next_n, width].
    """
    ctx = np.asarray(context_lens).tolist()
    B = len(ctx)
    out = np.full((B * next_n, width), np.nan, dtype=np.float64)
    want = set(range(B * next_n)) if rows is None else set(int(r) for r in rows)
    for b in range(B):
        todo = [j for j in range(next_n) if b * next_n + j in want]
        if not todo:
            continue
        c = ctx[b]
        nblk = -(-c // BLOCK)
        blocks = np.asarray(block_table[b][:nblk]).tolist()
        kc = np.concatenate([_block_values(cache, x) for x in blocks])[:c] if nblk else \
            np.zeros((0, DIM), np.uint8)
        ks = np.concatenate([_block_scales(cache, x) for x in blocks])[:c] if nblk else \
            np.zeros((0,), np.float32)
        for j in todo:
            r = b * next_n + j
            lim = c - next_n + j + 1
            row = np.full(width, -np.inf, dtype=np.float64)
            if lim > 0:
                row[:lim] = _score(q_codes[b, j], w[r], kc[:lim], ks[:lim])
            if not clean:
                row[nblk * BLOCK:] = np.nan
            out[r] = row
    return out


def mqa_logits(q_codes, w, k_codes, k_scale, cu_seq_lens, width, rows=None):
    """Prefill logits against contiguous (gathered) K, causal per request.

    The same score as ``paged_mqa_logits``; token p = cu[b] + i of request b
    sees the request's keys 0..i, and column j is the request-local key index
    (the K rows produced by ``gather_indexer_k``).  Later columns are -inf.
    q_codes: uint8 [total, H, D]; w: float32 [total, H]; k_codes uint8
    [total, D]; k_scale float32 [total].  Returns float64 [total, width];
    rows outside ``rows`` (if given) and rows of no request stay NaN.
    """
    cu = np.asarray(cu_seq_lens).tolist()
    total = q_codes.shape[0]
    out = np.full((total, width), np.nan, dtype=np.float64)
    want = set(range(total)) if rows is None else set(int(r) for r in rows)
    for b in range(len(cu) - 1):
        for p in range(cu[b], cu[b + 1]):
            if p not in want:
                continue
            lim = p - cu[b] + 1
            row = np.full(width, -np.inf, dtype=np.float64)
            row[:lim] = _score(q_codes[p], w[p], k_codes[cu[b]:cu[b] + lim],
                               k_scale[cu[b]:cu[b] + lim])
            out[p] = row
    return out


def mqa_logits_chunked(q_codes, w, k_codes, k_scale, cu_q, cu_k, width, rows=None):
    """Prefill logits of a chunk of each request's queries against the
    request's whole gathered context (chunked prefill; a ragged batch of
    such requests).

    Request b's queries are rows [cu_q[b], cu_q[b+1]) and its keys the K rows
    [cu_k[b], cu_k[b+1]) that ``gather_indexer_k`` writes with cu_k (ROCm/ATOM
    PR #1094, Technical Details, "sparse MLA prefill KV mapping"; vLLM PR
    #25869, the gather over cu_seq_lens).  The queries are the last
    n_q = cu_q[b+1] - cu_q[b] tokens of the request's n_k = cu_k[b+1] - cu_k[b]
    tokens, so query i sees keys [0, n_k - n_q + i + 1) -- the rule a decode
    request with next_n = n_q follows (reading R4); n_q = n_k is plain prefill.
    Column j is the request-local key index; later columns are -inf (all of
    them when n_k - n_q + i + 1 <= 0, a context shorter than its chunk).  A
    row whose limit exceeds ``width`` is not scored and stays NaN, like rows
    outside ``rows`` and rows of no request.
    """
    cq = np.asarray(cu_q).tolist()
    ck = np.asarray(cu_k).tolist()
    total = q_codes.shape[0]
    out = np.full((total, width), np.nan, dtype=np.float64)
    want = set(range(total)) if rows is None else set(int(r) for r in rows)
    for b in range(len(cq) - 1):
        n_q = cq[b + 1] - cq[b]
        n_k = ck[b + 1] - ck[b]
        for i in range(max(n_q, 0)):
            p = cq[b] + i
            lim = max(n_k - n_q + i + 1, 0)
            if p not in want or lim > width:
                continue
            row = np.full(width, -np.inf, dtype=np.float64)
            if lim > 0:
                row[:lim] = _score(q_codes[p], w[p], k_codes[ck[b]:ck[b] + lim],
                                   k_scale[ck[b]:ck[b] + lim])
            out[p] = row
    return out


# --------------------------------------------------------------------------
# top-k and slot ids
# --------------------------------------------------------------------------
def topk_rows(logits, row_len, k):
    """Per-row top-k over the visible columns, by a full sort.

    ROCm/ATOM PR #1094 (Technical Details) selects a sparse top-k per query
    and hands it on in a 2-D index buffer.  Column s < row_len[r] is ranked by
    the key (-L[r, s], s): larger logit first, lower index first among equal
    logits (-0.0 == +0.0).  A NaN ranks after every number (-inf included)
    and NaNs tie with each other (the pages print no rule for NaN; this is
    the ranking the library documents for the NaN logits of blocks outside
    the pool).  The first min(k, n) are written in ascending column order,
    then -1 padding.  Returns int32 [rows, k].
    """
    logits = np.asarray(logits)
    R, W = logits.shape
    out = np.full((R, k), -1, dtype=np.int32)
    for r in range(R):
        n = int(min(max(int(row_len[r]), 0), W))
        with np.errstate(invalid="ignore"):                 # signalling NaNs widen quietly
            vals = logits[r, :n].astype(np.float64) + 0.0  # -0.0 -> +0.0
        nan = np.isnan(vals)
        idx = np.arange(n)
        # by NaN last, then -value, then index
        order = np.lexsort((idx, -np.where(nan, 0.0, vals), nan))
        sel = np.sort(order[:min(k, n)])
        out[r, :sel.size] = sel
    return out


def topk_to_global_slots(topk_idx, row_req, block_table):
    """Request-local top-k indices -> global paged KV slot ids.

    ROCm/ATOM PR #1094 (Technical Details) converts the request-local top-k
    indices into global paged KV indices for sparse MLA decode; with 64-token
    blocks, local index i of request b lives in slot
    block_table[b][i // 64] * 64 + i % 64.  -1 (padding: no token) stays -1.
    An index the table does not map also gives -1: a row whose request is
    not a row of the table, an index whose block lies past the table's
    width, or a negative table entry (the table's own "no block" marker).
    """
    topk_idx = np.asarray(topk_idx)
    table_all = np.asarray(block_table, dtype=np.int64)
    n_req, n_cols = table_all.shape
    out = np.full(topk_idx.shape, -1, dtype=np.int32)
    for r in range(topk_idx.shape[0]):
        b = int(row_req[r])
        if b < 0 or b >= n_req:
            continue
        i = topk_idx[r].astype(np.int64)
        col = np.where(i >= 0, i // BLOCK, n_cols)
        mapped = col < n_cols
        blk = np.full(i.shape, -1, dtype=np.int64)
        blk[mapped] = table_all[b, col[mapped]]
        ok = mapped & (blk >= 0)
        out[r, ok] = (blk[ok] * BLOCK + i[ok] % BLOCK).astype(np.int32)
    return out
