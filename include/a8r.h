/*
 * a8r -- rolling-window decoder attention with exact RoPE re-basing, on MI355X.
 *
 * A cache holds, for every (layer, stream) pair, a ring of W key/value slots in
 * HBM.  Appending a token writes its K/V rows into the next slot; once W tokens
 * are live, each new token overwrites the oldest one (the pair that is evicted).
 * Attention rotates keys and queries on read, by their index counted from the
 * window's current origin (the oldest live token), so query-key distances are
 * exact however large the absolute positions grow.  The ring holds K and V
 * exactly as appended (a bit copy) and never modifies them.
 *
 * Passages this interface follows:
 *  - "Audio8 ASR Infinite: What It Actually Takes to Listen Forever", flowchart
 *    figure and section "Inside the Rolling KV Cache and Exact RoPE Re-Basing":
 *    fixed capacity, oldest-first eviction, re-basing of every surviving key's
 *    and the query's rotary index to the new origin, attention over the window,
 *    reset of the utterance state after a completed turn.
 *  - "Audio8-ASR-Infinite-mlx", section "Requires a patched mlx-audio-swift":
 *    split-half (rotate_half) rotary pairing.
 *  - "Audio8-ASR-0.1B in audio.cpp", section "Architecture": RoPE theta 1e6.
 *  - "Reza2kn/Audio8-ASR-Infinite-Compressed", sections "Linux CPU" and
 *    "Profile, provenance and integrity": the KV cache is stored in BF16.
 *  - Same blog, section "Semantic VAD: What the Decoder Predicts That Energy VAD
 *    Can't": the decoder advances once per audio clock of 80/120/160 ms, i.e.
 *    one or several new positions per call (the chunk path).
 *
 * Conventions for every call:
 *  - Errors are returned as a8r_status; nothing throws across the ABI.  Every
 *    argument check runs before any side effect, so a call that fails with
 *    A8R_EINVAL / A8R_ESTATE / A8R_EUNSUPPORTED changes no state.  A failing HIP
 *    call returns A8R_EDEVICE and poisons the cache: later calls on it return
 *    A8R_ESTATE.  a8r_last_error() describes the last failure of the calling
 *    thread.
 *  - "device" pointers are HIP device addresses (e.g. torch CUDA tensor
 *    data_ptr()); "host" pointers are ordinary CPU memory.  The caller owns all
 *    input/output buffers; the library owns the ring, its bookkeeping and its
 *    scratch unless a caller workspace is given at creation.
 *  - Device work is enqueued asynchronously on the cache's HIP stream in call
 *    order.  Device inputs must stay valid and unmodified until the stream has
 *    executed the call.  A cache is not thread-safe.
 *  - Element type of the ring and of every Q/K/V/O buffer is the config dtype
 *    (A8R_BF16: bf16 bit patterns, A8R_F32: float32).  Q/K/V/O device buffers
 *    must be 16-byte aligned and dense in the layouts stated per call.  K/V
 *    values must be finite.
 *  - Positions are int64; no absolute position is ever converted to floating
 *    point.  Rotation angles are formed from re-based indices < W + 32 only.
 */
#ifndef A8R_H
#define A8R_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum a8r_status {
    A8R_OK = 0,
    A8R_EINVAL = 1,        /* bad argument; nothing changed */
    A8R_ENOMEM = 2,        /* device allocation failed, or workspace too small */
    A8R_EDEVICE = 3,       /* a HIP call failed; the cache is now poisoned */
    A8R_ESTATE = 4,        /* call not valid in the current state (empty window, poisoned cache) */
    A8R_EUNSUPPORTED = 5   /* valid request this library does not implement */
} a8r_status;

typedef enum a8r_dtype { A8R_F32 = 0, A8R_BF16 = 1 } a8r_dtype;

/* Kernel selection.  AUTO picks the bf16 MFMA kernels where the shape allows
 * (bf16, head_dim 64 or 128; decode with <= 16 query heads per KV head; chunks
 * of 2..16 positions) and the portable kernels otherwise; PORTABLE forces the
 * portable kernels (used to cross-check the two). */
typedef enum a8r_kernel_policy { A8R_KERNELS_AUTO = 0, A8R_KERNELS_PORTABLE = 1 } a8r_kernel_policy;

/* How stored keys carry their rotation.
 *
 * A8R_ROTATE_ON_READ (the method): every read rotates a key by its re-based
 * index ("Audio8 ASR Infinite: What It Actually Takes to Listen Forever",
 * section "Inside the Rolling KV Cache and Exact RoPE Re-Basing": re-basing
 * every surviving key to the new origin keeps relative distances exact).
 * Keys and values are stored exactly as appended and never change, so nothing
 * accumulates.  A read at re-based index r applies R(r) in float32 with
 * coefficients from a table built in float64 and rounded once to float32
 * (the MFMA kernels split it as R(r - t) on the query and R(t) on the key,
 * t = the key's offset in its 32-slot tile, and round the rotated key once,
 * to the bf16 operand).
 *
 * A8R_REBASE_ON_EVICT (a comparison variant: the hazard the same page raises
 * there and in "Failure Modes That Only Appear on Day Three of a Session",
 * rounding error entering the rotation at every boundary): K is stored already
 * rotated to its re-based index, in the cache dtype, and whenever an append
 * evicts e tokens (the origin moves by e) every surviving key is re-rotated by
 * R(-e) and rounded back to the cache dtype.  Each re-rotation adds rounding
 * error that never leaves; it also reads and writes the whole K window at every
 * eviction.  The rotation arithmetic is float32 multiplies and adds without
 * fusion, rounded once to the cache dtype (round to nearest even).
 * Decode and chunk attention then use the stored keys as they are (the query is
 * still rotated by its re-based index).  The fused append + decode call runs as
 * the two separate steps in this mode. */
typedef enum a8r_cache_mode { A8R_ROTATE_ON_READ = 0, A8R_REBASE_ON_EVICT = 1 } a8r_cache_mode;

typedef struct a8r_config {
    int32_t n_layers;      /* >= 1 */
    int32_t n_streams;     /* >= 1; independent streams (batch) */
    int32_t n_q_heads;     /* >= 1, multiple of n_kv_heads */
    int32_t n_kv_heads;    /* >= 1; query head h uses KV head h / (n_q_heads / n_kv_heads) */
    int32_t head_dim;      /* 64 or 128 */
    int32_t window;        /* W >= 1: ring capacity in tokens per (layer, stream) */
    int32_t max_chunk;     /* 1 <= max_chunk <= W: most tokens per append / chunk call */
    int32_t dtype;         /* a8r_dtype */
    int32_t kernel_policy; /* a8r_kernel_policy */
    int32_t cache_mode;    /* a8r_cache_mode (0 = A8R_ROTATE_ON_READ) */
    double rope_theta;     /* > 0; frequencies theta^(-2i/head_dim), split-half pairs (i, i + head_dim/2) */
    float softmax_scale;   /* > 0, or <= 0 for 1/sqrt(head_dim) */
    float reserved_f;      /* must be 0 */
    int32_t prefix_capacity; /* >= 0: pinned prefix tokens per (layer, stream) besides the W ring
                                (see a8r_append_prefix); 0 = none */
    int32_t reserved;      /* must be 0 */
} a8r_config;

typedef struct a8r_cache a8r_cache;

/* Bytes of device memory a cache with this config needs (ring K and V, the
 * rotation table, per-pair state and split scratch), or 0 if cfg is invalid. */
size_t a8r_workspace_bytes(const a8r_config* cfg);

/* Create a cache.  cfg: host.  hip_stream: the hipStream_t all device work of
 * this cache is enqueued on (NULL = the default stream).  workspace: NULL to let
 * the library allocate, else a device buffer of ws_bytes >= a8r_workspace_bytes
 * bytes, 256-byte aligned, that the caller keeps alive until destroy.  The ring
 * and state are zeroed; every stream starts with P = 0 (next position),
 * L = 0 (live tokens), S = 0 (next slot).  *out receives the cache (host).
 * Errors: EINVAL (bad config or pointers), ENOMEM, EDEVICE (no usable device). */
a8r_status a8r_cache_create(const a8r_config* cfg, void* hip_stream, void* workspace,
                            size_t ws_bytes, a8r_cache** out);

/* Synchronize the cache's stream and release everything the library owns.
 * NULL is a no-op. */
void a8r_cache_destroy(a8r_cache* cache);

/* Change the stream later calls are enqueued on.  The caller orders the two
 * streams (e.g. with an event) if work is still pending on the old one. */
a8r_status a8r_set_stream(a8r_cache* cache, void* hip_stream);

/* Reset streams [b0, b0 + nb) in EVERY layer: L = 0, P = next_pos[i],
 * S = next_slot[i] (or next_pos[i] mod W when next_slot is NULL).  The window is
 * empty afterwards; old ring bytes are not cleared and are never read while not
 * live.  next_pos: host int64[nb], each >= 0; next_slot: host int32[nb] in
 * [0, W) or NULL.  Source: the blog's flowchart node "Emit final segment, reset
 * utterance state" (a reset after a completed turn or a silence restart).
 * Errors: EINVAL, ESTATE (poisoned), EDEVICE. */
a8r_status a8r_reset(a8r_cache* cache, int32_t b0, int32_t nb, const int64_t* next_pos,
                     const int32_t* next_slot);

/* Pinned prompt prefix.  A stream may hold up to prefix_capacity prefix tokens
 * that are never evicted, besides its W-token ring ("Audio8-ASR-Infinite-
 * Compressed", Linux CPU notes: an audio-independent prompt prefix prepared
 * once and re-checked at every silence reset).  The pages do not say how a
 * pinned prefix meets re-basing; the reading here: attention runs over the
 * sequence [prefix; live window] with consecutive re-based indices, so prefix
 * token j has index j, the window's live tokens F .. F + L - 1 (F = prefix
 * length), and a chunk's query c index F + L - C + c.  The prefix-to-query
 * distance therefore grows while the window fills and then stays fixed, like
 * every other distance in the window.
 *
 * a8r_append_prefix appends n_new tokens to the prefix of streams [b0, b0+nb)
 * in one layer.  k, v: device [nb][n_new][n_kv_heads][head_dim], 16-byte
 * aligned.  The stream's ring in that layer must be empty (L == 0: the prefix
 * precedes the window) and F + n_new <= prefix_capacity.  a8r_reset leaves
 * prefixes in place; a8r_clear_prefix empties them in every layer.  Not
 * available with A8R_REBASE_ON_EVICT (EUNSUPPORTED).
 * Errors: EINVAL, ESTATE (ring not empty, poisoned), EUNSUPPORTED, EDEVICE. */
a8r_status a8r_append_prefix(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb, int32_t n_new,
                             const void* k, const void* v);
/* Export and import of a prepared prefix (the pages prepare a prefix once, as
 * a separate operation, bound to the build and its configuration, and load it
 * for every session; "Audio8-ASR-Infinite-Compressed", Linux CPU notes).
 * a8r_export_prefix copies the n prefix tokens of streams [b0, b0+nb) in one
 * layer to k_out, v_out: device [nb][n][n_kv_heads][head_dim], 16-byte
 * aligned, K and V as appended (the bits a8r_append_prefix took).  Every
 * stream in the range must hold exactly n >= 1 prefix tokens.
 * a8r_import_prefix takes exactly that output (same head count, head_dim and
 * dtype) and appends it to the prefixes of streams [b0, b0+nb) bit for bit;
 * its preconditions and errors are a8r_append_prefix's.  An exported prefix
 * imported at the same prefix offset (e.g. into empty prefixes) reproduces the
 * original cache's stored bits.  Asynchronous on the cache's stream.
 * Errors: EINVAL, ESTATE, EUNSUPPORTED, EDEVICE. */
a8r_status a8r_export_prefix(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb, int32_t n,
                             void* k_out, void* v_out);
a8r_status a8r_import_prefix(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb, int32_t n_new,
                             const void* k, const void* v);
a8r_status a8r_clear_prefix(a8r_cache* cache, int32_t b0, int32_t nb);
/* Prefix length F of one (layer, stream) pair (host output). */
a8r_status a8r_prefix_length(a8r_cache* cache, int32_t layer, int32_t b, int32_t* length);

/* Append n_new tokens to streams [b0, b0 + nb) of one layer.  k, v: device,
 * [nb][n_new][n_kv_heads][head_dim], dtype elements.  Token j of stream b takes
 * position P + j and slot S; if L == W the token it replaces (position P + j - W)
 * is evicted; then S = (S + 1) mod W and L = min(L + 1, W); finally P += n_new.
 * slots_out (host int32[nb * n_new], or NULL) receives the slots and evicted_out
 * (host int64[nb * n_new], or NULL) the evicted positions (-1 = none), both
 * filled synchronously from the host-side bookkeeping before return.  The ring
 * write itself is asynchronous on the stream.  Source: the blog's flowchart
 * nodes "Rolling KV cache, fixed capacity" and "Evict oldest pair".
 * Errors: EINVAL (1 <= n_new <= max_chunk, ranges, null/misaligned k or v),
 * ESTATE, EDEVICE. */
a8r_status a8r_append_kv(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb, int32_t n_new,
                         const void* k, const void* v, int32_t* slots_out, int64_t* evicted_out);

/* Decode attention for the newest token of streams [b0, b0 + nb) of one layer.
 * q: device [nb][n_q_heads][head_dim]; out: device [nb][n_q_heads][head_dim].
 * The query is the last appended token; with origin o = P - L it has re-based
 * index L - 1 and attends to all L live keys (its own included), key at position
 * p having index p - o.  Both are rotated (split-half RoPE) by those indices;
 * out = softmax(scale * q_rot . k_rot) v per query head.  Source: the blog's
 * flowchart nodes "Shift sliding origin forward, re-base all remaining RoPE
 * indices to new zero" and "Attention over window", and section "Inside the
 * Rolling KV Cache and Exact RoPE Re-Basing".
 * Errors: EINVAL, ESTATE (some stream has L == 0, or poisoned), EDEVICE. */
a8r_status a8r_decode_attn(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb,
                           const void* q, void* out);

/* Attention for the last n_new appended tokens of streams [b0, b0 + nb) of one
 * layer (several positions per audio clock).  q, out: device
 * [nb][n_new][n_q_heads][head_dim].  Query c (0-based) has re-based index
 * L - n_new + c and sees keys with index <= its own: causal inside the chunk,
 * the whole older window before it.  Requires 1 <= n_new <= max_chunk and
 * n_new <= L for every stream.  Source: same passages as decode, plus the
 * blog's section "Semantic VAD: What the Decoder Predicts That Energy VAD
 * Can't" (80/120/160 ms clocks) and its note on leakage across chunk boundaries.
 * Errors: EINVAL, ESTATE (n_new > L for some stream, or poisoned), EDEVICE. */
a8r_status a8r_chunk_attn(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb,
                          int32_t n_new, const void* q, void* out);

/* a8r_chunk_attn for callers that cannot allocate device memory, or must not
 * depend on a workspace region: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, preconditions and
 * results as a8r_chunk_attn (bit for bit), except n_new >= 2; the kernels'
 * split partials live in one static device array of the library (64 MiB per
 * GPU, held until the process ends) instead of the cache's workspace.  A call
 * needs min(nb, 128) * n_kv_heads * 16 * n_new * group * (head_dim + 2) * 4
 * bytes of it (rounded up to 256 at the boundary of the two parts) when
 * n_new <= 16, none above; more than 64 MiB is rejected with EINVAL before any
 * side effect.  Allocates nothing (the array's address is looked up once per
 * device).  Every call on a GPU shares that GPU's array, which keeps the last
 * call's contents; calls that overlap on one GPU (other streams, other caches)
 * race and must be ordered by the caller.
 * Errors: as a8r_chunk_attn; EINVAL also for n_new < 2 or the size above. */
a8r_status a8r_chunk_attn_static(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb,
                                 int32_t n_new, const void* q, void* out);

/* The decode step of an audio clock in one call: exactly a8r_append_kv with
 * n_new = 1 followed by a8r_decode_attn on the same streams, executed as a
 * single kernel (the new token's K/V are written into the ring by the same
 * launch that attends to them).  k, v: device [nb][n_kv_heads][head_dim];
 * q, out: device [nb][n_q_heads][head_dim]; slots_out / evicted_out as for
 * a8r_append_kv (host, nb entries each, or NULL).  Shapes the fused kernel
 * does not cover (float32, head groups above 16) run as the two calls.
 * Errors: as a8r_append_kv and a8r_decode_attn; nothing changes on error. */
a8r_status a8r_append_decode_attn(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb, const void* k,
                                  const void* v, const void* q, void* out, int32_t* slots_out,
                                  int64_t* evicted_out);

/* The same for a chunk: exactly a8r_append_kv with n_new tokens followed by
 * a8r_chunk_attn with n_new queries on the same streams, as one launch where
 * the chunk kernel covers the shape (bfloat16, head_dim 64 or 128,
 * 2 <= n_new, n_new * group <= 128, keys not stored rotated to their index;
 * the block that owns a new token's 32-slot tile writes it before walking).
 * n_new = 1 is a8r_append_decode_attn.  k, v: device
 * [nb][n_new][n_kv_heads][head_dim]; q, out: device [nb][n_new][n_q_heads][head_dim];
 * slots_out / evicted_out: host [nb][n_new] or NULL.  Source: as
 * a8r_chunk_attn.  Errors: as a8r_append_kv and a8r_chunk_attn; nothing
 * changes on error. */
a8r_status a8r_append_chunk_attn(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb, int32_t n_new,
                                 const void* k, const void* v, const void* q, void* out, int32_t* slots_out,
                                 int64_t* evicted_out);

/* Window re-prefill, the comparison the scope table's last row asks for: the
 * window of streams [b0, b0+nb) in `layer` is rebuilt from stored hidden
 * states, the way "audio8-asr-infinite-p150" (section "Limitations") rebuilds
 * its decoder's rolling context by re-prefilling instead of trimming.  For each
 * stream, K = H Wk^T and V = H Wv^T over the n tokens of H:
 *   hidden: device [nb][n][hidden_dim] bf16, the window's tokens oldest first;
 *   w_k, w_v: device [n_kv_heads * head_dim][hidden_dim] bf16 (a linear
 *   layer's weight layout, no bias); output column kh * head_dim + d is
 *   element d of KV head kh.
 * Each result is a float32 accumulation of bf16 products rounded once to bf16
 * (nearest even).  The n tokens become the window: the positions P-n .. P-1
 * (P unchanged), token j in ring slot j, L = n, next slot n mod W; a pinned
 * prefix is kept.  16-byte aligned pointers, 1 <= n <= W, n <= P,
 * hidden_dim a multiple of 64 (at most 65536).  Asynchronous on the cache's
 * stream.  Errors: EINVAL, EUNSUPPORTED (float32 caches, A8R_REBASE_ON_EVICT,
 * n_kv_heads * head_dim not a multiple of 128, n * hidden_dim * 2 >= 2^31
 * bytes per stream), EDEVICE; nothing changes on error.  Slots of the last
 * 8-slot block past n (not live) are overwritten with token n - 1's V. */
a8r_status a8r_rebuild_window(a8r_cache* cache, int32_t layer, int32_t b0, int32_t nb, int32_t n,
                              int32_t hidden_dim, const void* hidden, const void* w_k, const void* w_v);

/* Read the state of one (layer, stream) pair: next position P, live count L,
 * next slot S (host outputs, any may be NULL).  Synchronizes the stream and
 * checks the device-side copy against the host bookkeeping; a mismatch returns
 * EDEVICE.  For tests and tooling. */
a8r_status a8r_get_state(a8r_cache* cache, int32_t layer, int32_t b, int64_t* next_pos,
                         int32_t* length, int32_t* next_slot);

/* Copy the ring of one (layer, stream) pair to host, in physical slot order, K
 * and V as appended (with A8R_REBASE_ON_EVICT keys rotated to their index):
 * k_host, v_host: host [W][n_kv_heads][head_dim] dtype elements (either may be
 * NULL).  Synchronizes the stream.  For tests and tooling. */
a8r_status a8r_read_ring(a8r_cache* cache, int32_t layer, int32_t b, void* k_host, void* v_host);

/* Description of the calling thread's last error ("" if none).  Valid until
 * the next a8r call on this thread. */
const char* a8r_last_error(void);

/* ---- host-only bookkeeping (the ring ledger), usable without a GPU -------- */
/* The same bookkeeping the cache runs on the host, exposed on its own so it can
 * be exercised and checked without a device.  Semantics as a8r_reset /
 * a8r_append_kv / a8r_get_state above.  All pointers are host pointers. */
typedef struct a8r_ledger a8r_ledger;

a8r_status a8r_ledger_create(int32_t n_layers, int32_t n_streams, int32_t window, a8r_ledger** out);
void a8r_ledger_destroy(a8r_ledger* ledger);
a8r_status a8r_ledger_reset(a8r_ledger* ledger, int32_t b0, int32_t nb, const int64_t* next_pos,
                            const int32_t* next_slot);
a8r_status a8r_ledger_append(a8r_ledger* ledger, int32_t layer, int32_t b0, int32_t nb,
                             int32_t n_new, int32_t* slots_out, int64_t* evicted_out);
a8r_status a8r_ledger_get(const a8r_ledger* ledger, int32_t layer, int32_t b, int64_t* next_pos,
                          int32_t* length, int32_t* next_slot);

/* Library version string, e.g. "a8r 0.1.0 gfx950". */
const char* a8r_version(void);

#ifdef __cplusplus
}
#endif

#endif /* A8R_H */
