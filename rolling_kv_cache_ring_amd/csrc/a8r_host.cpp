// Host side of the a8r C ABI: argument validation, the ring ledger (host copy
// of every (layer, stream) state), the float64 rotation-table builder, device
// memory layout, and the calls that enqueue the kernels.
//
// The ledger follows "Audio8 ASR Infinite: What It Actually Takes to Listen
// Forever", flowchart figure (fixed-capacity cache, "Evict oldest pair") and
// section "Inside the Rolling KV Cache and Exact RoPE Re-Basing": per pair the
// state (P, L, S) = (next absolute position, live tokens <= W, next slot); token
// j of an append takes slot S, evicts position P + j - W once L == W, then
// S = (S + 1) mod W, L = min(L + 1, W); P += n at the end.  The device keeps its
// own copy of the same state, advanced by the append kernel; a8r_get_state
// checks that both agree.

#include "a8r.h"

#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <limits>
#include <new>
#include <string>
#include <vector>

#include "a8r_internal.h"

namespace {

thread_local std::string g_last_error;

a8r_status fail(a8r_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

a8r_status ok() {
    g_last_error.clear();
    return A8R_OK;
}

struct PairState {
    int64_t next_pos;
    int32_t length;
    int32_t next_slot;
};

// Host bookkeeping for every (layer, stream) pair.
struct Ledger {
    int32_t n_layers = 0, n_streams = 0, window = 0;
    std::vector<PairState> st;

    void init(int32_t nl, int32_t ns, int32_t w) {
        n_layers = nl;
        n_streams = ns;
        window = w;
        st.assign((size_t)nl * ns, PairState{0, 0, 0});
    }
    PairState& at(int32_t layer, int32_t b) { return st[(size_t)layer * n_streams + b]; }
    const PairState& at(int32_t layer, int32_t b) const { return st[(size_t)layer * n_streams + b]; }

    // Checks an append of n_new tokens to streams [b0, b0+nb) can be admitted.
    a8r_status check_append(int32_t layer, int32_t b0, int32_t nb, int32_t n_new) const {
        if (layer < 0 || layer >= n_layers) return fail(A8R_EINVAL, "layer %d out of [0, %d)", layer, n_layers);
        if (nb < 1 || b0 < 0 || b0 > n_streams - nb)
            return fail(A8R_EINVAL, "streams [%d, %d+%d) out of [0, %d)", b0, b0, nb, n_streams);
        if (n_new < 1 || n_new > window) return fail(A8R_EINVAL, "n_new %d out of [1, W=%d]", n_new, window);
        for (int32_t i = 0; i < nb; ++i) {
            if (at(layer, b0 + i).next_pos > std::numeric_limits<int64_t>::max() - n_new)
                return fail(A8R_EINVAL, "stream %d: position would overflow int64", b0 + i);
        }
        return A8R_OK;
    }

    void append(int32_t layer, int32_t b0, int32_t nb, int32_t n_new, int32_t* slots, int64_t* evicted) {
        for (int32_t i = 0; i < nb; ++i) {
            PairState& s = at(layer, b0 + i);
            for (int32_t j = 0; j < n_new; ++j) {
                const size_t o = (size_t)i * n_new + j;
                if (slots) slots[o] = s.next_slot;
                if (evicted) evicted[o] = s.length == window ? s.next_pos + j - window : -1;
                s.next_slot = s.next_slot + 1 == window ? 0 : s.next_slot + 1;
                if (s.length < window) ++s.length;
            }
            s.next_pos += n_new;
        }
    }

    // Window rebuilt from n tokens (the last n positions, P unchanged), held in
    // slots 0 .. n-1.
    void rebuild(int32_t layer, int32_t b0, int32_t nb, int32_t n) {
        for (int32_t i = 0; i < nb; ++i) {
            PairState& s = at(layer, b0 + i);
            s.length = n;
            s.next_slot = n == window ? 0 : n;
        }
    }

    a8r_status check_reset(int32_t b0, int32_t nb, const int64_t* next_pos, const int32_t* next_slot) const {
        if (nb < 1 || b0 < 0 || b0 > n_streams - nb)
            return fail(A8R_EINVAL, "streams [%d, %d+%d) out of [0, %d)", b0, b0, nb, n_streams);
        if (!next_pos) return fail(A8R_EINVAL, "next_pos is NULL");
        for (int32_t i = 0; i < nb; ++i) {
            if (next_pos[i] < 0) return fail(A8R_EINVAL, "next_pos[%d] = %lld < 0", i, (long long)next_pos[i]);
            if (next_slot && (next_slot[i] < 0 || next_slot[i] >= window))
                return fail(A8R_EINVAL, "next_slot[%d] = %d out of [0, %d)", i, next_slot[i], window);
        }
        return A8R_OK;
    }

    void reset(int32_t b0, int32_t nb, const int64_t* next_pos, const int32_t* next_slot) {
        for (int32_t i = 0; i < nb; ++i) {
            const int32_t slot = next_slot ? next_slot[i] : (int32_t)(next_pos[i] % window);
            for (int32_t layer = 0; layer < n_layers; ++layer) at(layer, b0 + i) = PairState{next_pos[i], 0, slot};
        }
    }
};

struct Layout {
    size_t k_off, v_off, table_off, state_off, part_o_off, part_ml_off, part_x_off, total;
    int w_pad, f_pad, rows_max;
};

bool mul_ok(size_t a, size_t b, size_t* out) {
    if (a != 0 && b > std::numeric_limits<size_t>::max() / a) return false;
    *out = a * b;
    return true;
}

a8r_status validate_config(const a8r_config* c) {
    if (!c) return fail(A8R_EINVAL, "config is NULL");
    if (c->n_layers < 1) return fail(A8R_EINVAL, "n_layers %d < 1", c->n_layers);
    if (c->n_streams < 1) return fail(A8R_EINVAL, "n_streams %d < 1", c->n_streams);
    if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads)
        return fail(A8R_EINVAL, "n_q_heads %d must be a positive multiple of n_kv_heads %d", c->n_q_heads,
                    c->n_kv_heads);
    if (c->head_dim != 64 && c->head_dim != 128) return fail(A8R_EUNSUPPORTED, "head_dim %d (64 or 128)", c->head_dim);
    if (c->window < 1 || c->window > (1 << 28)) return fail(A8R_EINVAL, "window %d out of [1, 2^28]", c->window);
    if (c->max_chunk < 1 || c->max_chunk > c->window)
        return fail(A8R_EINVAL, "max_chunk %d out of [1, W=%d]", c->max_chunk, c->window);
    if (c->dtype != A8R_F32 && c->dtype != A8R_BF16) return fail(A8R_EINVAL, "dtype %d", c->dtype);
    if (c->kernel_policy != A8R_KERNELS_AUTO && c->kernel_policy != A8R_KERNELS_PORTABLE)
        return fail(A8R_EINVAL, "kernel_policy %d", c->kernel_policy);
    if (c->cache_mode != A8R_ROTATE_ON_READ && c->cache_mode != A8R_REBASE_ON_EVICT)
        return fail(A8R_EINVAL, "cache_mode %d", c->cache_mode);
    if (c->reserved_f != 0.f || c->reserved != 0) return fail(A8R_EINVAL, "reserved fields must be 0");
    if (c->prefix_capacity < 0 || c->prefix_capacity > (1 << 20))
        return fail(A8R_EINVAL, "prefix_capacity %d out of [0, 2^20]", c->prefix_capacity);
    if (c->prefix_capacity > 0 && c->cache_mode == A8R_REBASE_ON_EVICT)
        return fail(A8R_EUNSUPPORTED, "a pinned prefix is not available with A8R_REBASE_ON_EVICT");
    if (!(c->rope_theta > 0.0) || !isfinite(c->rope_theta)) return fail(A8R_EINVAL, "rope_theta must be > 0");
    if (!isfinite(c->softmax_scale)) return fail(A8R_EINVAL, "softmax_scale must be finite");
    if ((int64_t)c->n_q_heads * (int64_t)c->n_streams > (1 << 24))
        return fail(A8R_EINVAL, "n_q_heads * n_streams too large");
    return A8R_OK;
}

a8r_status compute_layout(const a8r_config* c, Layout* lay) {
    const size_t eb = c->dtype == A8R_BF16 ? 2 : 4;
    const int w_pad = (int)((c->window + a8r::kTile - 1) / a8r::kTile * a8r::kTile);
    const int group = c->n_q_heads / c->n_kv_heads;
    const int qmax = c->max_chunk < a8r::kMaxPartialQ ? c->max_chunk : a8r::kMaxPartialQ;
    const int rows_max = qmax * group;
    const int f_pad = (int)((c->prefix_capacity + a8r::kTile - 1) / a8r::kTile * a8r::kTile);
    size_t pairs, ring, t;
    if (!mul_ok((size_t)c->n_layers * c->n_streams, (size_t)c->n_kv_heads, &pairs) ||
        !mul_ok(pairs, (size_t)(w_pad + f_pad) * c->head_dim, &t) || !mul_ok(t, eb, &ring))
        return fail(A8R_EINVAL, "ring size overflows size_t");
    // rows up to W + f_pad: a query at most W - 1 + F indices past a prefix tile
    const size_t table = (size_t)(c->window + f_pad + a8r::kTablePad) * (c->head_dim / 2) * 8;
    const size_t state = (size_t)c->n_layers * c->n_streams * sizeof(a8r::DevState);
    const size_t prow = (size_t)c->n_streams * c->n_kv_heads * a8r::kMaxSplits * rows_max;
    size_t off = 0;
    lay->k_off = off;
    off = a8r::align_up(off + ring, a8r::kAlign);
    lay->v_off = off;
    off = a8r::align_up(off + ring, a8r::kAlign);
    lay->table_off = off;
    off = a8r::align_up(off + table, a8r::kAlign);
    lay->state_off = off;
    off = a8r::align_up(off + state, a8r::kAlign);
    lay->part_o_off = off;
    off = a8r::align_up(off + prow * c->head_dim * 4, a8r::kAlign);
    lay->part_ml_off = off;
    off = a8r::align_up(off + prow * 2 * 4, a8r::kAlign);
    lay->part_x_off = off;
    off = a8r::align_up(off + (size_t)c->n_streams * c->n_kv_heads * a8r::kXSlots * a8r::kMaxGroupMfma *
                                  c->head_dim * sizeof(uint64_t),
                        a8r::kAlign);
    lay->total = off;
    lay->w_pad = w_pad;
    lay->f_pad = f_pad;
    lay->rows_max = rows_max;
    return A8R_OK;
}

// (cos, sin)(r * theta^(-2i/D)) for r < W + 32, i < D/2, computed in float64
// and rounded once to float32.  Split-half pairing (i, i + D/2) per
// "Audio8-ASR-Infinite-mlx", section "Requires a patched mlx-audio-swift";
// theta per "Audio8-ASR-0.1B in audio.cpp", section "Architecture".  Row r is
// the rotation for re-based index r; indices are always small (< W + 32), so
// the float64 angle is exact to ~1e-16 relative.
std::vector<float> build_table(int window, int f_pad, int head_dim, double theta) {
    const int np = head_dim / 2;
    const int rows = window + f_pad + a8r::kTablePad;
    std::vector<double> inv(np);
    for (int i = 0; i < np; ++i) inv[i] = pow(theta, -2.0 * i / head_dim);
    std::vector<float> t((size_t)rows * np * 2);
    for (int r = 0; r < rows; ++r) {
        for (int i = 0; i < np; ++i) {
            const double a = (double)r * inv[i];
            t[((size_t)r * np + i) * 2] = (float)cos(a);
            t[((size_t)r * np + i) * 2 + 1] = (float)sin(a);
        }
    }
    return t;
}

}  // namespace

struct a8r_cache {
    a8r_config cfg{};
    Ledger ledger;
    Layout lay{};
    a8r::Geometry geo{};
    hipStream_t stream = nullptr;
    void* base = nullptr;
    std::vector<int32_t> prefix;  // pinned prefix length per (layer, stream)
    bool owns = false;
    bool poisoned = false;
    int device = 0;
    int n_cu = 256;
};

struct a8r_ledger {
    Ledger l;
};

namespace {

a8r_status device_fail(a8r_cache* c, hipError_t e, const char* what) {
    if (c) c->poisoned = true;
    return fail(A8R_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

a8r_status check_live(const a8r_cache* c) {
    if (!c) return fail(A8R_EINVAL, "cache is NULL");
    if (c->poisoned) return fail(A8R_ESTATE, "cache is poisoned by an earlier device error");
    return A8R_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

a8r_status check_streams(const a8r_cache* c, int32_t layer, int32_t b0, int32_t nb) {
    if (layer < 0 || layer >= c->cfg.n_layers) return fail(A8R_EINVAL, "layer %d out of [0, %d)", layer, c->cfg.n_layers);
    if (nb < 1 || b0 < 0 || b0 > c->cfg.n_streams - nb)
        return fail(A8R_EINVAL, "streams [%d, %d+%d) out of [0, %d)", b0, b0, nb, c->cfg.n_streams);
    return A8R_OK;
}

}  // namespace

extern "C" {

const char* a8r_last_error(void) { return g_last_error.c_str(); }

const char* a8r_version(void) { return "a8r 0.1.0 gfx950"; }

size_t a8r_workspace_bytes(const a8r_config* cfg) {
    if (validate_config(cfg) != A8R_OK) return 0;
    Layout lay;
    if (compute_layout(cfg, &lay) != A8R_OK) return 0;
    return lay.total;
}

a8r_status a8r_cache_create(const a8r_config* cfg, void* hip_stream, void* workspace, size_t ws_bytes,
                            a8r_cache** out) {
    if (!out) return fail(A8R_EINVAL, "out is NULL");
    *out = nullptr;
    a8r_status st = validate_config(cfg);
    if (st != A8R_OK) return st;
    Layout lay;
    if ((st = compute_layout(cfg, &lay)) != A8R_OK) return st;
    if (workspace && ws_bytes < lay.total)
        return fail(A8R_ENOMEM, "workspace of %zu bytes < %zu needed", ws_bytes, lay.total);
    if (workspace && ((uintptr_t)workspace % a8r::kAlign))
        return fail(A8R_EINVAL, "workspace must be %zu-byte aligned", a8r::kAlign);

    a8r_cache* c = new (std::nothrow) a8r_cache();
    if (!c) return fail(A8R_ENOMEM, "host allocation failed");
    c->cfg = *cfg;
    c->lay = lay;
    c->stream = (hipStream_t)hip_stream;
    c->ledger.init(cfg->n_layers, cfg->n_streams, cfg->window);
    c->prefix.assign((size_t)cfg->n_layers * cfg->n_streams, 0);

    hipError_t e = hipGetDevice(&c->device);
    if (e != hipSuccess) {
        delete c;
        return fail(A8R_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    }
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, c->device) == hipSuccess && ncu > 0)
        c->n_cu = ncu;
    if (workspace) {
        c->base = workspace;
    } else {
        e = hipMalloc(&c->base, lay.total);
        if (e != hipSuccess) {
            delete c;
            return fail(A8R_ENOMEM, "hipMalloc(%zu): %s", lay.total, hipGetErrorString(e));
        }
        c->owns = true;
    }
    uint8_t* b = (uint8_t*)c->base;
    a8r::Geometry& g = c->geo;
    g.k_ring = b + lay.k_off;
    g.v_ring = b + lay.v_off;
    g.table = (const float2*)(b + lay.table_off);
    g.state = (a8r::DevState*)(b + lay.state_off);
    g.part_o = (float*)(b + lay.part_o_off);
    g.part_ml = (float*)(b + lay.part_ml_off);
    g.part_x = (uint64_t*)(b + lay.part_x_off);
    g.n_layers = cfg->n_layers;
    g.n_streams = cfg->n_streams;
    g.hq = cfg->n_q_heads;
    g.hkv = cfg->n_kv_heads;
    g.group = cfg->n_q_heads / cfg->n_kv_heads;
    g.d = cfg->head_dim;
    g.window = cfg->window;
    g.w_pad = lay.w_pad;
    g.f_pad = lay.f_pad;
    g.pair_slots = lay.w_pad + lay.f_pad;
    g.elem_bytes = cfg->dtype == A8R_BF16 ? 2 : 4;
    g.prerot = cfg->cache_mode == A8R_REBASE_ON_EVICT;
    g.rows_max = lay.rows_max;
    const double scale = cfg->softmax_scale > 0.f ? (double)cfg->softmax_scale : 1.0 / sqrt((double)cfg->head_dim);
    g.scale_log2 = (float)(scale * 1.4426950408889634);  // log2(e)

    const std::vector<float> table = build_table(cfg->window, lay.f_pad, cfg->head_dim, cfg->rope_theta);
    e = hipMemsetAsync(c->base, 0, lay.total, c->stream);
    if (e == hipSuccess)   // every exchange slot starts empty (all ones)
        e = hipMemsetAsync(b + lay.part_x_off, 0xff, lay.total - lay.part_x_off, c->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(b + lay.table_off, table.data(), table.size() * sizeof(float), hipMemcpyHostToDevice,
                           c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) {
        if (c->owns) (void)hipFree(c->base);
        delete c;
        return fail(A8R_EDEVICE, "cache initialisation: %s", hipGetErrorString(e));
    }
    *out = c;
    return ok();
}

void a8r_cache_destroy(a8r_cache* c) {
    if (!c) return;
    (void)hipStreamSynchronize(c->stream);
    if (c->owns && c->base) (void)hipFree(c->base);
    delete c;
}

a8r_status a8r_set_stream(a8r_cache* c, void* hip_stream) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    c->stream = (hipStream_t)hip_stream;
    return ok();
}

}  // extern "C"

namespace {

// Fills the launch-argument state of streams [b0, b0 + nb) of one layer from
// the host bookkeeping.
void fill_batch(const a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, a8r::StreamBatch* sb) {
    sb->b0 = b0;
    sb->nb = nb;
    for (int32_t i = 0; i < nb; ++i) {
        const PairState& p = c->ledger.at(layer, b0 + i);
        sb->next_slot[i] = p.next_slot;
        sb->length[i] = p.length;
        sb->prefix[i] = c->prefix[(size_t)layer * c->cfg.n_streams + b0 + i];
        sb->next_pos[i] = p.next_pos;
    }
}

}  // namespace

extern "C" {

a8r_status a8r_reset(a8r_cache* c, int32_t b0, int32_t nb, const int64_t* next_pos, const int32_t* next_slot) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = c->ledger.check_reset(b0, nb, next_pos, next_slot)) != A8R_OK) return st;
    std::vector<int32_t> slots(nb);
    for (int32_t i = 0; i < nb; ++i)
        slots[i] = next_slot ? next_slot[i] : (int32_t)(next_pos[i] % c->cfg.window);
    c->ledger.reset(b0, nb, next_pos, slots.data());
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, 0, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        hipError_t e = a8r::launch_reset(c->geo, sb, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "reset kernel");
    }
    return ok();
}

a8r_status a8r_append_kv(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_new, const void* k,
                         const void* v, int32_t* slots_out, int64_t* evicted_out) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = c->ledger.check_append(layer, b0, nb, n_new)) != A8R_OK) return st;
    if (n_new > c->cfg.max_chunk) return fail(A8R_EINVAL, "n_new %d > max_chunk %d", n_new, c->cfg.max_chunk);
    if (!k || !v) return fail(A8R_EINVAL, "k or v is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(A8R_EINVAL, "k and v must be 16-byte aligned");
    const size_t row = (size_t)n_new * c->cfg.n_kv_heads * c->cfg.head_dim * c->geo.elem_bytes;
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, layer, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        hipError_t e = a8r::launch_append(c->geo, layer, sb, n_new, (const uint8_t*)k + i0 * row,
                                          (const uint8_t*)v + i0 * row, c->stream);
        if (e == hipSuccess && c->geo.prerot) e = a8r::launch_rebase(c->geo, layer, sb, n_new, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "append kernel");
    }
    c->ledger.append(layer, b0, nb, n_new, slots_out, evicted_out);
    return ok();
}

static a8r_status check_attention(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_q, int32_t added,
                                  const void* q, void* out) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = check_streams(c, layer, b0, nb)) != A8R_OK) return st;
    if (n_q < 1 || n_q > c->cfg.max_chunk)
        return fail(A8R_EINVAL, "n_new %d out of [1, max_chunk=%d]", n_q, c->cfg.max_chunk);
    if (!q || !out) return fail(A8R_EINVAL, "q or out is NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(A8R_EINVAL, "q and out must be 16-byte aligned");
    for (int32_t i = 0; i < nb; ++i) {
        const int32_t len = std::min(c->ledger.at(layer, b0 + i).length + added, c->cfg.window);
        if (len < n_q)
            return fail(A8R_ESTATE, "stream %d layer %d holds %d live tokens, need >= %d", b0 + i, layer, len,
                        n_q);
    }
    return A8R_OK;
}

static a8r_status attention_call(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_q, const void* q,
                                  void* out) {
    a8r_status st = check_attention(c, layer, b0, nb, n_q, 0, q, out);
    if (st != A8R_OK) return st;
    const size_t qrow = (size_t)n_q * c->cfg.n_q_heads * c->cfg.head_dim * c->geo.elem_bytes;
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, layer, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        hipError_t e = a8r::launch_attention(c->geo, layer, sb, n_q, (const uint8_t*)q + i0 * qrow,
                                             (uint8_t*)out + i0 * qrow, c->cfg.kernel_policy == A8R_KERNELS_AUTO,
                                             c->n_cu, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "attention kernel");
    }
    return ok();
}

a8r_status a8r_decode_attn(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, const void* q, void* out) {
    return attention_call(c, layer, b0, nb, 1, q, out);
}

a8r_status a8r_chunk_attn(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_new, const void* q,
                          void* out) {
    return attention_call(c, layer, b0, nb, n_new, q, out);
}

a8r_status a8r_chunk_attn_static(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_new,
                                 const void* q, void* out) {
    a8r_status st = check_attention(c, layer, b0, nb, n_new, 0, q, out);
    if (st != A8R_OK) return st;
    if (n_new < 2) return fail(A8R_EINVAL, "n_new %d < 2 (one query per stream is a8r_decode_attn)", n_new);
    // split partials of one launch (up to kBatch streams), laid out as the
    // cache's own: [stream][kv head][kMaxSplits][row][D] float32, then (m, l)
    const a8r::Geometry& cg = c->geo;
    const size_t rows = (size_t)n_new * cg.group;
    const size_t nbl = (size_t)std::min(nb, a8r::kBatch);
    const size_t o_bytes =
        a8r::align_up(nbl * cg.hkv * a8r::kMaxSplits * rows * cg.d * sizeof(float), a8r::kAlign);
    const size_t need = n_new <= a8r::kMaxPartialQ ? o_bytes + nbl * cg.hkv * a8r::kMaxSplits * rows * 2 * sizeof(float)
                                                   : 0;
    if (need > a8r::kStaticScratchBytes)
        return fail(A8R_EINVAL,
                    "a8r_chunk_attn_static: %d streams x %d KV heads x %d query rows need %zu bytes of split "
                    "partials, more than the %zu-byte static scratch (use fewer streams per call)",
                    (int)nbl, cg.hkv, (int)rows, need, a8r::kStaticScratchBytes);
    void* base = nullptr;
    hipError_t e = a8r::static_scratch(c->device, &base);
    if (e != hipSuccess) return fail(A8R_EDEVICE, "static scratch address: %s", hipGetErrorString(e));
    a8r::Geometry g = cg;
    g.rows_max = (int)rows;
    g.part_o = (float*)base;
    g.part_ml = (float*)((uint8_t*)base + o_bytes);
    const size_t qrow = (size_t)n_new * c->cfg.n_q_heads * c->cfg.head_dim * c->geo.elem_bytes;
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, layer, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        e = a8r::launch_attention(g, layer, sb, n_new, (const uint8_t*)q + i0 * qrow, (uint8_t*)out + i0 * qrow,
                                  c->cfg.kernel_policy == A8R_KERNELS_AUTO, c->n_cu, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "attention kernel");
    }
    return ok();
}

a8r_status a8r_append_decode_attn(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, const void* k,
                                  const void* v, const void* q, void* out, int32_t* slots_out,
                                  int64_t* evicted_out) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = c->ledger.check_append(layer, b0, nb, 1)) != A8R_OK) return st;
    if (!k || !v) return fail(A8R_EINVAL, "k or v is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(A8R_EINVAL, "k and v must be 16-byte aligned");
    if ((st = check_attention(c, layer, b0, nb, 1, 1, q, out)) != A8R_OK) return st;
    const size_t kvrow = (size_t)c->cfg.n_kv_heads * c->cfg.head_dim * c->geo.elem_bytes;
    const size_t qrow = (size_t)c->cfg.n_q_heads * c->cfg.head_dim * c->geo.elem_bytes;
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, layer, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        hipError_t e = a8r::launch_append_decode(c->geo, layer, sb, (const uint8_t*)k + i0 * kvrow,
                                                 (const uint8_t*)v + i0 * kvrow, (const uint8_t*)q + i0 * qrow,
                                                 (uint8_t*)out + i0 * qrow,
                                                 c->cfg.kernel_policy == A8R_KERNELS_AUTO, c->n_cu, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "append+decode kernel");
    }
    c->ledger.append(layer, b0, nb, 1, slots_out, evicted_out);
    return ok();
}

a8r_status a8r_append_chunk_attn(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_new,
                                 const void* k, const void* v, const void* q, void* out, int32_t* slots_out,
                                 int64_t* evicted_out) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = c->ledger.check_append(layer, b0, nb, n_new)) != A8R_OK) return st;
    if (n_new > c->cfg.max_chunk) return fail(A8R_EINVAL, "n_new %d > max_chunk %d", n_new, c->cfg.max_chunk);
    if (!k || !v) return fail(A8R_EINVAL, "k or v is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(A8R_EINVAL, "k and v must be 16-byte aligned");
    if ((st = check_attention(c, layer, b0, nb, n_new, n_new, q, out)) != A8R_OK) return st;
    const size_t kvrow = (size_t)n_new * c->cfg.n_kv_heads * c->cfg.head_dim * c->geo.elem_bytes;
    const size_t qrow = (size_t)n_new * c->cfg.n_q_heads * c->cfg.head_dim * c->geo.elem_bytes;
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, layer, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        hipError_t e = a8r::launch_append_chunk(c->geo, layer, sb, n_new, (const uint8_t*)k + i0 * kvrow,
                                                (const uint8_t*)v + i0 * kvrow, (const uint8_t*)q + i0 * qrow,
                                                (uint8_t*)out + i0 * qrow,
                                                c->cfg.kernel_policy == A8R_KERNELS_AUTO, c->n_cu, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "append+chunk kernel");
    }
    c->ledger.append(layer, b0, nb, n_new, slots_out, evicted_out);
    return ok();
}

a8r_status a8r_rebuild_window(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n, int32_t hidden_dim,
                              const void* hidden, const void* w_k, const void* w_v) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = check_streams(c, layer, b0, nb)) != A8R_OK) return st;
    if (c->geo.elem_bytes != 2) return fail(A8R_EUNSUPPORTED, "window rebuild needs a bf16 cache");
    if (c->geo.prerot) return fail(A8R_EUNSUPPORTED, "window rebuild is not available with A8R_REBASE_ON_EVICT");
    if ((c->geo.hkv * c->geo.d) % 128)
        return fail(A8R_EUNSUPPORTED, "window rebuild needs n_kv_heads * head_dim %% 128 == 0 (got %d)",
                    c->geo.hkv * c->geo.d);
    if (n < 1 || n > c->cfg.window) return fail(A8R_EINVAL, "n %d out of [1, W=%d]", n, c->cfg.window);
    if (hidden_dim < 64 || hidden_dim % 64 || hidden_dim > (1 << 16))
        return fail(A8R_EINVAL, "hidden_dim %d must be a positive multiple of 64, at most 65536", hidden_dim);
    if ((int64_t)n * hidden_dim * 2 >= ((int64_t)1 << 31))   // the kernel's 32-bit offsets into one stream's rows
        return fail(A8R_EUNSUPPORTED, "window rebuild needs n * hidden_dim * 2 < 2^31 bytes per stream (got %lld)",
                    (long long)n * hidden_dim * 2);
    if (!hidden || !w_k || !w_v) return fail(A8R_EINVAL, "hidden, w_k or w_v is NULL");
    if (!aligned16(hidden) || !aligned16(w_k) || !aligned16(w_v))
        return fail(A8R_EINVAL, "hidden, w_k and w_v must be 16-byte aligned");
    for (int32_t i = 0; i < nb; ++i)
        if (c->ledger.at(layer, b0 + i).next_pos < n)
            return fail(A8R_EINVAL, "stream %d layer %d: next position %lld < n = %d (window before position 0)",
                        b0 + i, layer, (long long)c->ledger.at(layer, b0 + i).next_pos, n);
    const size_t row = (size_t)n * hidden_dim * 2;
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, layer, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        hipError_t e = a8r::launch_rebuild(c->geo, layer, sb, n, hidden_dim, (const uint8_t*)hidden + i0 * row,
                                           w_k, w_v, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "window rebuild kernel");
    }
    c->ledger.rebuild(layer, b0, nb, n);
    return ok();
}

static a8r_status append_prefix(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_new, const void* k,
                                const void* v) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = check_streams(c, layer, b0, nb)) != A8R_OK) return st;
    if (c->cfg.prefix_capacity == 0) return fail(A8R_EUNSUPPORTED, "the cache has no prefix capacity");
    if (n_new < 1) return fail(A8R_EINVAL, "n_new %d < 1", n_new);
    if (!k || !v) return fail(A8R_EINVAL, "k or v is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(A8R_EINVAL, "k and v must be 16-byte aligned");
    for (int32_t i = 0; i < nb; ++i) {
        const size_t at = (size_t)layer * c->cfg.n_streams + b0 + i;
        if (c->ledger.at(layer, b0 + i).length != 0)
            return fail(A8R_ESTATE, "stream %d layer %d: the prefix must precede the window (L = %d)", b0 + i,
                        layer, c->ledger.at(layer, b0 + i).length);
        if (c->prefix[at] + n_new > c->cfg.prefix_capacity)
            return fail(A8R_EINVAL, "stream %d layer %d: prefix %d + %d exceeds capacity %d", b0 + i, layer,
                        c->prefix[at], n_new, c->cfg.prefix_capacity);
    }
    const size_t row = (size_t)n_new * c->cfg.n_kv_heads * c->cfg.head_dim * c->geo.elem_bytes;
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, layer, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        hipError_t e = a8r::launch_append_prefix(c->geo, layer, sb, n_new, (const uint8_t*)k + i0 * row,
                                                 (const uint8_t*)v + i0 * row, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "prefix append kernel");
    }
    for (int32_t i = 0; i < nb; ++i) c->prefix[(size_t)layer * c->cfg.n_streams + b0 + i] += n_new;
    return ok();
}

a8r_status a8r_append_prefix(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_new, const void* k,
                             const void* v) {
    return append_prefix(c, layer, b0, nb, n_new, k, v);
}

a8r_status a8r_import_prefix(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n_new, const void* k,
                             const void* v) {
    return append_prefix(c, layer, b0, nb, n_new, k, v);
}

a8r_status a8r_export_prefix(a8r_cache* c, int32_t layer, int32_t b0, int32_t nb, int32_t n, void* k, void* v) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = check_streams(c, layer, b0, nb)) != A8R_OK) return st;
    if (n < 1) return fail(A8R_EINVAL, "n %d < 1", n);
    if (!k || !v) return fail(A8R_EINVAL, "k or v is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(A8R_EINVAL, "k and v must be 16-byte aligned");
    for (int32_t i = 0; i < nb; ++i) {
        const int32_t f = c->prefix[(size_t)layer * c->cfg.n_streams + b0 + i];
        if (f != n) return fail(A8R_EINVAL, "stream %d layer %d: prefix length %d, not %d", b0 + i, layer, f, n);
    }
    const size_t row = (size_t)n * c->cfg.n_kv_heads * c->cfg.head_dim * c->geo.elem_bytes;
    for (int32_t i0 = 0; i0 < nb; i0 += a8r::kBatch) {
        a8r::StreamBatch sb;
        fill_batch(c, layer, b0 + i0, std::min(a8r::kBatch, nb - i0), &sb);
        hipError_t e = a8r::launch_export_prefix(c->geo, layer, sb, n, (uint8_t*)k + i0 * row,
                                                 (uint8_t*)v + i0 * row, c->stream);
        if (e != hipSuccess) return device_fail(c, e, "prefix export kernel");
    }
    return ok();
}

a8r_status a8r_clear_prefix(a8r_cache* c, int32_t b0, int32_t nb) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = check_streams(c, 0, b0, nb)) != A8R_OK) return st;
    for (int32_t layer = 0; layer < c->cfg.n_layers; ++layer)
        for (int32_t i = 0; i < nb; ++i) c->prefix[(size_t)layer * c->cfg.n_streams + b0 + i] = 0;
    return ok();
}

a8r_status a8r_prefix_length(a8r_cache* c, int32_t layer, int32_t b, int32_t* length) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = check_streams(c, layer, b, 1)) != A8R_OK) return st;
    if (!length) return fail(A8R_EINVAL, "length is NULL");
    *length = c->prefix[(size_t)layer * c->cfg.n_streams + b];
    return ok();
}

a8r_status a8r_get_state(a8r_cache* c, int32_t layer, int32_t b, int64_t* next_pos, int32_t* length,
                         int32_t* next_slot) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = check_streams(c, layer, b, 1)) != A8R_OK) return st;
    a8r::DevState ds;
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e == hipSuccess)
        e = hipMemcpy(&ds, c->geo.state + (size_t)layer * c->cfg.n_streams + b, sizeof ds, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return device_fail(c, e, "state readback");
    const PairState& h = c->ledger.at(layer, b);
    if (next_pos) *next_pos = h.next_pos;
    if (length) *length = h.length;
    if (next_slot) *next_slot = h.next_slot;
    if (ds.next_pos != h.next_pos || ds.length != h.length || ds.next_slot != h.next_slot)
        return fail(A8R_EDEVICE,
                    "device state (%lld, %d, %d) != host bookkeeping (%lld, %d, %d) for layer %d stream %d",
                    (long long)ds.next_pos, ds.length, ds.next_slot, (long long)h.next_pos, h.length, h.next_slot,
                    layer, b);
    return ok();
}

a8r_status a8r_read_ring(a8r_cache* c, int32_t layer, int32_t b, void* k_host, void* v_host) {
    a8r_status st = check_live(c);
    if (st != A8R_OK) return st;
    if ((st = check_streams(c, layer, b, 1)) != A8R_OK) return st;
    const a8r::Geometry& g = c->geo;
    const size_t eb = g.elem_bytes, D = g.d, W = g.window, wp = g.pair_slots, H = g.hkv;
    const size_t per_head = wp * D * eb;
    std::vector<uint8_t> tmp(per_head * H);
    hipError_t e = hipStreamSynchronize(c->stream);
    const size_t first = (size_t)a8r::pair_index(g, layer, b, 0);
    for (int pass = 0; pass < 2 && e == hipSuccess; ++pass) {
        void* dst = pass == 0 ? k_host : v_host;
        if (!dst) continue;
        const uint8_t* src = (const uint8_t*)(pass == 0 ? g.k_ring : g.v_ring) + first * per_head;
        e = hipMemcpy(tmp.data(), src, per_head * H, hipMemcpyDeviceToHost);
        if (e != hipSuccess) break;
        uint8_t* o = (uint8_t*)dst;
        for (size_t h = 0; h < H; ++h) {
            const uint8_t* t = tmp.data() + h * per_head;
            for (size_t s = 0; s < W; ++s) {
                for (size_t d = 0; d < D; ++d) {
                    const size_t from = pass == 0 ? (s * D + d) : (((s / 8) * D + d) * 8 + s % 8);
                    memcpy(o + ((s * H + h) * D + d) * eb, t + from * eb, eb);
                }
            }
        }
    }
    if (e != hipSuccess) return device_fail(c, e, "ring readback");
    return ok();
}

// ---- host-only ledger --------------------------------------------------------
a8r_status a8r_ledger_create(int32_t n_layers, int32_t n_streams, int32_t window, a8r_ledger** out) {
    if (!out) return fail(A8R_EINVAL, "out is NULL");
    *out = nullptr;
    if (n_layers < 1 || n_streams < 1 || window < 1)
        return fail(A8R_EINVAL, "n_layers, n_streams and window must be >= 1");
    a8r_ledger* l = new (std::nothrow) a8r_ledger();
    if (!l) return fail(A8R_ENOMEM, "host allocation failed");
    l->l.init(n_layers, n_streams, window);
    *out = l;
    return ok();
}

void a8r_ledger_destroy(a8r_ledger* l) { delete l; }

a8r_status a8r_ledger_reset(a8r_ledger* l, int32_t b0, int32_t nb, const int64_t* next_pos,
                            const int32_t* next_slot) {
    if (!l) return fail(A8R_EINVAL, "ledger is NULL");
    a8r_status st = l->l.check_reset(b0, nb, next_pos, next_slot);
    if (st != A8R_OK) return st;
    l->l.reset(b0, nb, next_pos, next_slot);
    return ok();
}

a8r_status a8r_ledger_append(a8r_ledger* l, int32_t layer, int32_t b0, int32_t nb, int32_t n_new,
                             int32_t* slots_out, int64_t* evicted_out) {
    if (!l) return fail(A8R_EINVAL, "ledger is NULL");
    a8r_status st = l->l.check_append(layer, b0, nb, n_new);
    if (st != A8R_OK) return st;
    l->l.append(layer, b0, nb, n_new, slots_out, evicted_out);
    return ok();
}

a8r_status a8r_ledger_get(const a8r_ledger* l, int32_t layer, int32_t b, int64_t* next_pos, int32_t* length,
                          int32_t* next_slot) {
    if (!l) return fail(A8R_EINVAL, "ledger is NULL");
    if (layer < 0 || layer >= l->l.n_layers || b < 0 || b >= l->l.n_streams)
        return fail(A8R_EINVAL, "pair (%d, %d) out of range", layer, b);
    const PairState& s = l->l.at(layer, b);
    if (next_pos) *next_pos = s.next_pos;
    if (length) *length = s.length;
    if (next_slot) *next_slot = s.next_slot;
    return ok();
}

}  // extern "C"
