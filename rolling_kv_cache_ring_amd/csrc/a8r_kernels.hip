// HIP kernels for rolling-window attention with exact RoPE re-basing (gfx950).
//
// Method ("Audio8 ASR Infinite: What It Actually Takes to Listen Forever",
// flowchart figure and section "Inside the Rolling KV Cache and Exact RoPE
// Re-Basing"): a ring of W slots per (layer, stream, KV head); the live window
// is the last L <= W tokens; its origin is the oldest live token.  A key at
// re-based index r and the query at index r_q are rotated (split-half RoPE,
// "Audio8-ASR-Infinite-mlx", section "Requires a patched mlx-audio-swift";
// theta from "Audio8-ASR-0.1B in audio.cpp", section "Architecture") on read;
// the stored K/V bits are never rewritten.  K and V are stored exactly as
// appended (a bit copy); every read rotates the key by its re-based index.
//
// Kernels:
//   reset_kernel       device record of the per-pair state after a reset
//   append_kernel      copies new K/V rows into their ring slots (one block
//                      per stream) and records the new state
//   attn_portable      any dtype / group size / chunk size; LDS-tiled VALU
//   combine_kernel     merges split-K partials {m, l, O} of attn_portable,
//                      and chunk_pipe
//   decode_mfma        bf16 decode (optionally fused with the append of the
//                      new token); QK^T and PV on v_mfma_f32_16x16x32_bf16,
//                      split-K partials merged inside the kernel (a fixed
//                      binary tree of per-element atomic exchanges)
//   chunk_pipe         bf16 chunks of 2..16 positions (query rows of a KV head
//                      in groups of up to 128 per block): keys rotated once
//                      per visit into an LDS tile, QK^T and PV on MFMA,
//                      software-pipelined
//   prefix_append_kernel, prefix_export_kernel
//                      a pinned prompt prefix (never evicted, attended before
//                      the window) into and out of its slots after the ring
//   rebase_kernel      the rebase-on-evict comparison variant's re-rotation
//
// The attention kernels take the prefix as extra tiles after the ring's; the
// prefix walk is a template flag, instantiated only for batches that hold one.
//
// Every kernel takes the ring state of its streams from its launch arguments
// (StreamBatch, filled by the host from its bookkeeping when the call is made).
// Scores are kept in base-2 units (the softmax scale is multiplied by log2 e)
// so every exponential is one v_exp_f32.

#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <type_traits>
#include <stdint.h>
#include <stdlib.h>

#include "a8r_internal.h"

namespace a8r {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;   // running-max seed: exp2(x - kNegBig) never NaNs

// 2^x as the single hardware instruction (v_exp_f32): arguments here are <= 8,
// and results below 2^-126 flush to 0, which is harmless for softmax weights.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max and sum over the lanes l, l^16, l^32, l^48 (the four lanes holding one
// MFMA output column) with gfx950's lane-swap instructions: each swap returns
// {x[l], x[l^16]} (resp. l^32) in some order, in VALU, without the LDS round
// trip of a bpermute.  Both operations are commutative, so every lane of the
// group gets the same bits.
__device__ __forceinline__ float max_rows4(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_rows4(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned w = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bf16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

template <int EB>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
    if constexpr (EB == 2) {
        return bf16_bits_to_f32(((const uint16_t*)base)[i]);
    } else {
        return ((const float*)base)[i];
    }
}

template <int EB>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float x) {
    if constexpr (EB == 2) {
        ((uint16_t*)base)[i] = f32_to_bf16_bits(x);
    } else {
        ((float*)base)[i] = x;
    }
}

__device__ __forceinline__ int wrap_slot(int s, int w) { return s >= w ? s - w : s; }

// ---------------------------------------------------------------- reset ----
__global__ void reset_kernel(Geometry g, StreamBatch r) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= g.n_layers * r.nb) return;
    const int layer = t / r.nb, i = t - layer * r.nb;
    DevState s;
    s.next_pos = r.next_pos[i];
    s.length = r.length[i];
    s.next_slot = r.next_slot[i];
    g.state[(int64_t)layer * g.n_streams + r.b0 + i] = s;
}

// --------------------------------------------------------------- append ----
// Writes one 16-byte chunk c of a token row of K and V into ring slot `slot`:
// K rows are row-major; element d of V for slot s lives at ((s/8)*D + d)*8 + s%8
// of the head's V block array.
template <int EB>
__device__ __forceinline__ void store_token(void* k_base, void* v_base, int pad, int D, int64_t pair, int slot,
                                            int c, u32x4 kv, u32x4 vv) {
    constexpr int per16 = 16 / EB;
    uint8_t* kdst = (uint8_t*)k_base + ((pair * pad + slot) * D + (int64_t)c * per16) * EB;
    *(u32x4*)kdst = kv;
    uint8_t* vblk = (uint8_t*)v_base + ((pair * (pad / 8) + slot / 8) * (int64_t)D * 8) * EB;
    const int lane8 = slot & 7;
#pragma unroll
    for (int u = 0; u < per16; ++u) {
        const int d = c * per16 + u;
        if constexpr (EB == 2) {
            const uint32_t w = vv[u >> 1];
            ((uint16_t*)vblk)[(int64_t)d * 8 + lane8] = (uint16_t)((u & 1) ? (w >> 16) : (w & 0xffffu));
        } else {
            ((uint32_t*)vblk)[(int64_t)d * 8 + lane8] = vv[u];
        }
    }
}

template <int EB>
__device__ __forceinline__ void write_token_vals(const Geometry& g, int64_t pair, int slot, int c, u32x4 kv,
                                                 u32x4 vv) {
    store_token<EB>(g.k_ring, g.v_ring, g.pair_slots, g.d, pair, slot, c, kv, vv);
}

// Copies 16-byte chunk c of one token's K and V rows (input layout
// [nb][n][Hkv][D]) into `slot` of a pair, bit for bit.
template <int EB>
__device__ __forceinline__ void write_token_chunk(const Geometry& g, int64_t pair, int slot, int c,
                                                  const uint8_t* krow, const uint8_t* vrow) {
    write_token_vals<EB>(g, pair, slot, c, *(const u32x4*)(krow + c * 16), *(const u32x4*)(vrow + c * 16));
}

// One block per stream; token j of stream b goes to slot (S + j) mod W.
template <int EB>
__global__ __launch_bounds__(256) void append_kernel(Geometry g, int layer, StreamBatch st, int n_new,
                                                     const uint8_t* __restrict__ k,
                                                     const uint8_t* __restrict__ v) {
    const int bi = blockIdx.x, b = st.b0 + bi;
    const int D = g.d, W = g.window;
    constexpr int per16 = 16 / EB;
    const int chunks = D / per16;                      // 16-byte chunks per row
    const int total = n_new * g.hkv * chunks;
    const int s0 = st.next_slot[bi];
    for (int t = threadIdx.x; t < total; t += blockDim.x) {
        const int c = t % chunks;
        const int rest = t / chunks;
        const int kh = rest % g.hkv, j = rest / g.hkv;
        const int64_t src = (((int64_t)bi * n_new + j) * g.hkv + kh) * D * EB;
        write_token_chunk<EB>(g, pair_index(g, layer, b, kh), wrap_slot(s0 + j, W), c, k + src, v + src);
    }
    if (threadIdx.x == 0) {
        DevState ns;
        ns.next_pos = st.next_pos[bi] + n_new;
        ns.length = min(st.length[bi] + n_new, W);
        ns.next_slot = wrap_slot(s0 + n_new, W);
        g.state[(int64_t)layer * g.n_streams + b] = ns;
    }
}

// Pinned prefix: token j of stream b goes to prefix slot F + j (pair slot
// w_pad + F + j, after the ring; never evicted), copied bit for bit like a
// ring token.  An import of a8r_export_prefix's output is the same copy.
template <int EB>
__global__ __launch_bounds__(256) void prefix_append_kernel(Geometry g, int layer, StreamBatch st, int n_new,
                                                            const uint8_t* __restrict__ k,
                                                            const uint8_t* __restrict__ v) {
    const int bi = blockIdx.x, b = st.b0 + bi;
    const int D = g.d;
    constexpr int per16 = 16 / EB;
    const int chunks = D / per16;
    const int total = n_new * g.hkv * chunks;
    const int f0 = st.prefix[bi];
    for (int t = threadIdx.x; t < total; t += blockDim.x) {
        const int c = t % chunks;
        const int rest = t / chunks;
        const int kh = rest % g.hkv, j = rest / g.hkv;
        const int64_t src = (((int64_t)bi * n_new + j) * g.hkv + kh) * D * EB;
        write_token_chunk<EB>(g, pair_index(g, layer, b, kh), g.w_pad + f0 + j, c, k + src, v + src);
    }
}

// Export of a pinned prefix: prefix token j of stream b back to row j of the
// append layout [nb][n][Hkv][D]: K rows as stored (the appended bits), V
// gathered back out of its transposed 8-slot blocks.  An import
// (prefix_append_kernel) restores exactly these bits.
template <int EB>
__global__ __launch_bounds__(256) void prefix_export_kernel(Geometry g, int layer, StreamBatch st, int n,
                                                            uint8_t* __restrict__ k, uint8_t* __restrict__ v) {
    const int bi = blockIdx.x, b = st.b0 + bi;
    const int D = g.d;
    constexpr int per16 = 16 / EB;
    const int chunks = D / per16;
    const int total = n * g.hkv * chunks;
    for (int t = threadIdx.x; t < total; t += blockDim.x) {
        const int c = t % chunks;
        const int rest = t / chunks;
        const int kh = rest % g.hkv, j = rest / g.hkv;
        const int64_t dst = ((((int64_t)bi * n + j) * g.hkv + kh) * D + (int64_t)c * per16) * EB;
        const int64_t pair = pair_index(g, layer, b, kh);
        const int slot = g.w_pad + j;
        *(u32x4*)(k + dst) =
            *(const u32x4*)((const uint8_t*)g.k_ring + ((pair * g.pair_slots + slot) * D + (int64_t)c * per16) * EB);
        const uint8_t* vblk =
            (const uint8_t*)g.v_ring + ((pair * (g.pair_slots / 8) + slot / 8) * (int64_t)D * 8) * EB;
        const int lane8 = slot & 7;
        u32x4 vv;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if constexpr (EB == 2) {
                const int d = c * per16 + 2 * u;
                const uint32_t lo = ((const uint16_t*)vblk)[(int64_t)d * 8 + lane8];
                const uint32_t hi = ((const uint16_t*)vblk)[(int64_t)(d + 1) * 8 + lane8];
                vv[u] = lo | (hi << 16);
            } else {
                vv[u] = ((const uint32_t*)vblk)[(int64_t)(c * per16 + u) * 8 + lane8];
            }
        }
        *(u32x4*)(v + dst) = vv;
    }
}

// ------------------------------------------------------ rebase on evict ----
// A8R_REBASE_ON_EVICT (a comparison variant): keys are stored rotated to their
// re-based index.  After an append of n tokens to a window of L0 keys (state
// `before`), the window holds L1 = min(L0 + n, W) keys and its origin moved by
// e = L0 + n - L1: the new tokens (indices L1 - n .. L1 - 1, written unrotated
// by append_kernel) are rotated by R(r), and every surviving key by
// R(-e) = R(e) conjugated.  Each pair is computed with float32 multiplies and
// adds without fusion and rounded once to the cache dtype, so the rounding of
// every re-rotation stays in the stored key.  Block = (256 keys of the window,
// KV head, stream); a thread takes one pair (i, i + D/2) of one key.
template <int D, int EB>
__global__ __launch_bounds__(256) void rebase_kernel(Geometry g, int layer, StreamBatch before, int n) {
    constexpr int NP = D / 2;
    const int bi = blockIdx.z, kh = blockIdx.y, r0 = blockIdx.x * 256;
    const int b = before.b0 + bi, W = g.window;
    const int L0 = before.length[bi];
    const int L1 = min(L0 + n, W), e = L0 + n - L1;
    int oldest = (before.next_slot[bi] + n - L1) % W;  // in (-W, W)
    if (oldest < 0) oldest += W;
    const int r_new = L1 - n;
    const int r_begin = e > 0 ? r0 : max(r0, r_new);   // without an eviction only new keys change
    const int r_end = min(r0 + 256, L1);
    if (r_begin >= r_end) return;
    uint8_t* kring = (uint8_t*)g.k_ring + pair_index(g, layer, b, kh) * g.pair_slots * D * EB;
    const int cnt = (r_end - r_begin) * NP;
    for (int t = threadIdx.x; t < cnt; t += 256) {
#pragma clang fp contract(off)
        const int r = r_begin + t / NP, i = t % NP;
        const int64_t at = (int64_t)wrap_slot(oldest + r, W) * D + i;
        float2 cs = g.table[(int64_t)(r >= r_new ? r : e) * NP + i];
        if (r < r_new) cs.y = -cs.y;
        const float x1 = load_elem<EB>(kring, at), x2 = load_elem<EB>(kring, at + NP);
        const float a = x1 * cs.x, b2 = x2 * cs.y, c2 = x2 * cs.x, d2 = x1 * cs.y;
        store_elem<EB>(kring, at, a - b2);
        store_elem<EB>(kring, at + NP, c2 + d2);
    }
}

// ------------------------------------------------------ split partials ----
__device__ __forceinline__ int64_t part_row(const Geometry& g, int bi, int kh, int split, int row) {
    return (((int64_t)bi * g.hkv + kh) * kMaxSplits + split) * g.rows_max + row;
}

// Merges the splits' partials: 256 threads, each 4 consecutive dims of one
// output row (stream, query, head); D/4 threads per row.  Every split's loads
// are issued together (one round trip), then combined in split order.
template <int D, int EB, int NS>
__global__ __launch_bounds__(256) void combine_kernel(Geometry g, int n_q, int n_split, void* out, int rows) {
    constexpr int TPR = D / 4, RPB = 256 / TPR;          // threads per row, rows per block
    const int o = blockIdx.x * RPB + threadIdx.x / TPR;
    const int d4 = threadIdx.x % TPR;
    if (o >= rows) return;
    const int h = o % g.hq;
    const int c = (o / g.hq) % n_q;
    const int bi = o / (g.hq * n_q);
    const int kh = h / g.group, row = c * g.group + (h - kh * g.group);
    // Every load unconditional (a split past n_split re-reads the last one and
    // gets weight 0) and at most NS (8 or 16) splits, so that they can all be
    // in flight at once (with a branch per split the compiler waited for each
    // split's loads before issuing the next).  The splits are merged online in
    // split order, each split's m, l and O used together, so no load is held
    // back behind arithmetic on the others.
    float mv[NS], lv[NS];
    float4 ov[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t pr = part_row(g, bi, kh, s < n_split ? s : n_split - 1, row);
        const floatx2 ml = __builtin_nontemporal_load((const floatx2*)&g.part_ml[pr * 2]);   // read once
        mv[s] = ml.x;
        lv[s] = ml.y;
        const floatx4 ox = __builtin_nontemporal_load((const floatx4*)&g.part_o[pr * D + 4 * d4]);
        ov[s] = float4{ox[0], ox[1], ox[2], ox[3]};
    }
    __builtin_amdgcn_sched_barrier(0);                 // every load issued before the merge
    float mmax = mv[0], den = lv[0];
    float4 num = ov[0];
#pragma unroll
    for (int s = 1; s < NS; ++s) {
        const bool live = s < n_split;                 // branch-free: past n_split a no-op
        const float mn = live ? fmaxf(mmax, mv[s]) : mmax;
        const float a = exp2f(mmax - mn), w = live ? exp2f(mv[s] - mn) : 0.f;
        den = den * a + lv[s] * w;
        num.x = num.x * a + ov[s].x * w;
        num.y = num.y * a + ov[s].y * w;
        num.z = num.z * a + ov[s].z * w;
        num.w = num.w * a + ov[s].w * w;
        mmax = mn;
    }
    const int64_t ob = (((int64_t)bi * n_q + c) * g.hq + h) * D + 4 * d4;
    store_elem<EB>(out, ob, num.x / den);
    store_elem<EB>(out, ob + 1, num.y / den);
    store_elem<EB>(out, ob + 2, num.z / den);
    store_elem<EB>(out, ob + 3, num.w / den);
}

template <int D, int EB>
hipError_t launch_combine(const Geometry& g, int nb, int n_q, int n_split, void* out, hipStream_t s) {
    constexpr int RPB = 256 / (D / 4);
    const int rows = nb * n_q * g.hq;
    auto kern = n_split <= 8 ? combine_kernel<D, EB, 8> : combine_kernel<D, EB, kMaxSplits>;
    hipLaunchKernelGGL(kern, dim3((rows + RPB - 1) / RPB), dim3(256), 0, s, g, n_q, n_split, out, rows);
    return hipGetLastError();
}

// --------------------------------------------------------- portable path ----
// Block = (split of the key range, KV head, stream) x (group of 64 query rows).
// Rows are (query c, head-in-group hg) = c * G + hg.  Keys are walked in
// re-based order r = 0 .. L-1 (slot = (oldest + r) mod W) in tiles of 16; each
// tile's K rows are rotated by R(r) into LDS (table row r; the conjugate of row
// |r| for a prefix key, r < 0); scores, online softmax and PV run
// on VALU with 4 threads per row (4 keys of the tile each for the scores, a
// quarter of the head dims each for PV).
template <int D, int EB>
__global__ __launch_bounds__(256) void attn_portable(Geometry g, int layer, StreamBatch st, int n_q,
                                                     const void* __restrict__ q,
                                                     void* __restrict__ out, int n_split) {
    constexpr int KT = 16, RG = 64, NP = D / 2, DQ = D / 4;
    __shared__ float qs[RG][D + 1];
    __shared__ float ks[KT][D + 1];
    __shared__ float vs[KT][D + 1];
    __shared__ float ps[RG][KT + 1];
    const int tid = threadIdx.x;
    const int bi = blockIdx.z, kh = blockIdx.y;
    const int split = blockIdx.x % n_split, rg = blockIdx.x / n_split;
    const int b = st.b0 + bi, G = g.group, W = g.window;
    const int rows = n_q * G, row0 = rg * RG;
    const int L = st.length[bi];
    int oldest = st.next_slot[bi] - L;
    if (oldest < 0) oldest += W;
    const int64_t pair = pair_index(g, layer, b, kh);
    const void* kring = (const uint8_t*)g.k_ring + pair * g.pair_slots * D * EB;
    const void* vring = (const uint8_t*)g.v_ring + pair * g.pair_slots * D * EB;
    // the pinned prefix (F tokens, pair slots w_pad ..) precedes the window: key
    // index r in [-F, L)
    const int F = st.prefix[bi];

    // rotated, scaled queries: query c has re-based index L - n_q + c
    for (int idx = tid; idx < RG * NP; idx += 256) {
        const int row = idx / NP, i = idx - row * NP, r = row0 + row;
        float y1 = 0.f, y2 = 0.f;
        if (r < rows) {
            const int c = r / G, h = kh * G + (r - c * G);
            const int rq = L - n_q + c;
            const int64_t qoff = (((int64_t)bi * n_q + c) * g.hq + h) * D;
            const float x1 = load_elem<EB>(q, qoff + i) * g.scale_log2;
            const float x2 = load_elem<EB>(q, qoff + i + NP) * g.scale_log2;
            const float2 cs = g.table[(int64_t)rq * NP + i];
            y1 = x1 * cs.x - x2 * cs.y;
            y2 = x2 * cs.x + x1 * cs.y;
        }
        qs[row][i] = y1;
        qs[row][i + NP] = y2;
    }

    const int my_row = tid >> 2, sub = tid & 3;
    const int r_glob = row0 + my_row;
    const bool row_ok = r_glob < rows;
    const int my_rq = row_ok ? L - n_q + r_glob / G : -1;
    float m = kNegBig, l = 0.f;
    float o[DQ];
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[i] = 0.f;

    const int n_kt = (F + L + KT - 1) / KT;
    const int per = (n_kt + n_split - 1) / n_split;
    const int kt0 = split * per, kt1 = min(n_kt, kt0 + per);
    for (int kt = kt0; kt < kt1; ++kt) {
        __syncthreads();
        for (int idx = tid; idx < KT * NP; idx += 256) {
            const int j = idx / NP, i = idx - j * NP, r = kt * KT + j - F;
            float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
            if (r < L) {
                // prefix token r + F (r < 0) at pair slot w_pad + r + F, else a ring slot
                const int slot = r < 0 ? g.w_pad + r + F : wrap_slot(oldest + r, W);
                const float x1 = load_elem<EB>(kring, (int64_t)slot * D + i);
                const float x2 = load_elem<EB>(kring, (int64_t)slot * D + i + NP);
                // R(r), the conjugate of row |r| for a prefix key (r < 0); keys
                // stored rotated to their index (A8R_REBASE_ON_EVICT) are used as they are
                float2 cs = g.prerot ? float2{1.f, 0.f} : g.table[(int64_t)(r < 0 ? -r : r) * NP + i];
                if (r < 0) cs.y = -cs.y;
                k1 = x1 * cs.x - x2 * cs.y;
                k2 = x2 * cs.x + x1 * cs.y;
                const int64_t vb = (int64_t)(slot >> 3) * D * 8 + (slot & 7);
                v1 = load_elem<EB>(vring, vb + (int64_t)i * 8);
                v2 = load_elem<EB>(vring, vb + (int64_t)(i + NP) * 8);
            }
            ks[j][i] = k1;
            ks[j][i + NP] = k2;
            vs[j][i] = v1;
            vs[j][i + NP] = v2;
        }
        __syncthreads();
        float s[4];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = sub * 4 + jj, r = kt * KT + j - F;
            float acc = 0.f;
            for (int d = 0; d < D; ++d) acc += qs[my_row][d] * ks[j][d];
            s[jj] = (row_ok && r < L && r <= my_rq) ? acc : -INFINITY;
            mx = fmaxf(mx, s[jj]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        const float m_new = fmaxf(m, mx);
        const float alpha = exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < DQ; ++i) o[i] *= alpha;
        m = m_new;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float p = exp2f(s[jj] - m);
            l += p;
            ps[my_row][sub * 4 + jj] = p;
        }
        __syncthreads();
        for (int j = 0; j < KT; ++j) {
            const float p = ps[my_row][j];
#pragma unroll
            for (int i = 0; i < DQ; ++i) o[i] += p * vs[j][sub * DQ + i];
        }
    }
    l += __shfl_xor(l, 1);
    l += __shfl_xor(l, 2);
    if (!row_ok) return;
    const int c = r_glob / G, hg = r_glob - c * G, h = kh * G + hg;
    if (n_split == 1) {
        const int64_t ob = (((int64_t)bi * n_q + c) * g.hq + h) * D + sub * DQ;
#pragma unroll
        for (int i = 0; i < DQ; ++i) store_elem<EB>(out, ob + i, o[i] / l);
    } else {
        const int64_t pr = part_row(g, bi, kh, split, r_glob);
#pragma unroll
        for (int i = 0; i < DQ; ++i) g.part_o[pr * D + sub * DQ + i] = o[i];
        if (sub == 0) {
            g.part_ml[pr * 2] = m;
            g.part_ml[pr * 2 + 1] = l;
        }
    }
}

// ------------------------------------------------------------ MFMA decode ----
// bf16 decode for one (stream, KV head, split) per block of 8 waves.
//
// The ring is walked in physical 32-slot tiles ("visits"), starting with the
// tile that holds the oldest live slot.  A visit's keys sit at slots s0 + t,
// t in [0, 32); their re-based indices are rho + t for one per-visit rho (the
// first visit may also hold the window's newest keys just before the oldest
// slot: those have index rho + t + W).
//
// Rotation: with R(x) the split-half rotation by index x, the score is
// <R(r_q) q, R(rho + t) k> = <R(r_q - rho) q, R(t) k> because rotations in each
// 2-D plane compose additively and are orthogonal.  The ring holds the keys as
// appended; a lane always reads the same two offsets t of a tile (its MFMA
// rows): the block stages the table rows R(t), t < 32, in LDS once, and each
// lane rotates its two key rows by theirs on every visit (float32, one
// rounding to the bf16 MFMA operand), while the query is rotated once per visit by
// R(r_q - rho), a table row (< W + 32) fetched with the visit's keys.  On the
// first visit the newest keys (offsets before the oldest slot, index
// rho + t + W) take a second query rotation R(r_q - rho - W), composed in
// float32 from that row and the R(W) row, and their scores are selected from
// it.  Every coefficient comes from the float64-built table; no absolute
// position enters float arithmetic.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, lane l = 16*gq + n):
//   QK: S^T[key][head] = K_rot[key][dims] * Q_rot^T; A row n of tile half b is
//       key t = 8*(n/4) + 4*b + n%4, so the result gives lane l the scores of
//       keys 8*gq .. 8*gq+7 for head n -- exactly the B operand of PV.
//   PV: O^T[d][head] = V^T[d][keys] * P^T; the A operand is 8 consecutive slots
//       of one dim, i.e. 16 bytes of the transposed 8-slot V block.
// Columns n >= G (padding) carry a copy of head 0 and are discarded.
//
// Memory pipeline: every global read of the kernel is a direct global->LDS
// load (global_load_lds_dwordx4, 16 bytes per lane at LDS base + 16*lane), so
// data in flight holds no registers.  Each wave owns one visit buffer, split
// in a K part (32 rows, whole cache lines per instruction, XOR-swizzled for
// conflict-free MFMA operand reads, plus the visit's query-rotation row) and a
// V part.  The scores of visit k wait only for K(k), its PV only for V(k), and
// each part is refilled with the wave's next visit (k + 8) as soon as it has
// been read.  Two waves share each SIMD, so one wave's rotation, MFMA and
// softmax work runs while the other waits for its loads (with one wave per
// SIMD and two buffers each, the key rotation could not hide behind the
// loads: 19.3 against 11.9 us for one 3B stream's layer).  The waits are explicit
// vmcnt counts; the DMA destinations are hidden from the compiler's own wait
// insertion (see opaque_lds), which would otherwise drain the queue.
//
// The splits of one (stream, KV head) merge their {m, l, O} partials per
// output element through atomic-exchange slots arranged in a fixed binary tree
// (see the end of the kernel).
//
// Fused append: with k_new != nullptr the state in the arguments is the state
// before the append, the window is the one after it, and the wave that owns
// the new token's tile patches the token into its LDS copy of that tile and
// writes it into its ring slot after the walk (no other wave or block reads
// that slot in the same launch).

// A raw buffer resource over `bytes` bytes at `base`: buffer loads take a
// 32-bit per-lane offset plus a scalar offset, and reads past the end return
// zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

struct DecodeCtx {
    const uint16_t* kp;
    const uint16_t* vp;
    const float2* table;
    rsrc_t kr, vr, tr;     // the pair's K and V blocks and the table, as buffers
    uint32_t koff[2];      // this lane's byte offsets inside a tile's K rows (loads j with
                           // ((64 j / (D/8)) >> 3) even, odd; a load's rows add 1024 j)
    uint32_t voff, toff;   // ... inside a tile's V blocks, and inside a table row
    int oldest, t_o, p0t, n_tiles, L, W, rq, tb0, tb1, gq, n;
    int n_roll, F;     // visits over the ring, then ceil(F / 32) over the prefix
    int pre_on;        // a pinned prefix may exist (compile-time in every kernel: without it
                       // the visit walk has no prefix branch)
    int prerot;        // keys stored rotated to their index: only the query is rotated
    float scale_log2;
};

__device__ __forceinline__ int visit_tile(const DecodeCtx& c, int k) {
    const int p = c.p0t + k;
    return p >= c.n_tiles ? p - c.n_tiles : p;
}

__device__ __forceinline__ int visit_rho(const DecodeCtx& c, int k, int s0) {
    if (k == 0) return -c.t_o;
    const int rho = s0 - c.oldest;
    return rho < 0 ? rho + c.W : rho;
}

// Where visit k reads from: the ring's tiles first (k < n_roll), then the pinned
// prefix's tiles, stored after the ring (tile n_tiles + m holds prefix tokens
// 32m .. 32m + 31, those below F live).  Relative to the window's origin a
// prefix token's re-based index is 32m + t - F < 0: the prefix sits just
// before the window (indices taken over [prefix; window]).  s0 is the tile's
// first slot, or for a prefix tile its first prefix token.
struct VisitSrc {
    int tile, s0, rho;
    bool pre;
};

__device__ __forceinline__ VisitSrc visit_src(const DecodeCtx& c, int k) {
    VisitSrc v;
    v.pre = c.pre_on && k >= c.n_roll;
    if (!v.pre) {
        v.tile = visit_tile(c, k);
        v.s0 = v.tile * kTile;
        v.rho = visit_rho(c, k, v.s0);
    } else {
        v.s0 = (k - c.n_roll) * kTile;
        v.tile = c.n_tiles + k - c.n_roll;
        v.rho = v.s0 - c.F;
    }
    return v;
}

// (cos, sin) of the lane's 8*(D/64) pairs (dims 8*gq + 32*kk + e, kk < D/64)
// of a table row staged in LDS.
template <int D>
__device__ __forceinline__ void lds_coef(const unsigned char* row, int gq, float4 (&cf)[D / 64][4]) {
    const float4* p = (const float4*)row + 4 * gq;
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) cf[kk][j] = p[16 * kk + j];
}

// The same from the block's copy of table rows 0 .. 31 (R(t) for a tile's key
// t), row t's 16-byte chunk col at chunk position (D/4) t + (col ^ k_swz(t)):
// the eight rows t of one read instruction's consecutive lanes then fall on
// distinct banks.
__device__ __forceinline__ int k_swz(int r);

template <int D>
__device__ __forceinline__ void lds_coef_t(const unsigned char* rows, int t, int gq, float4 (&cf)[D / 64][4]) {
    const float4* p = (const float4*)rows + (D / 4) * t;
    const int sw = k_swz(t);
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) cf[kk][j] = p[(4 * gq + 16 * kk + j) ^ sw];
}

// Rotates a lane's slice of a bf16 row (dims 8*gq + 32*kk + e) by the pairs in
// cf: x_i, x_{i+D/2} -> x_i c - x_{i+D/2} s, x_{i+D/2} c + x_i s, rounded to bf16.
template <int D>
__device__ __forceinline__ void rotate_row(const float4 (&cf)[D / 64][4], const u32x4 (&x)[D / 32],
                                           bf16x8 (&y)[D / 32]) {
    constexpr int HP = D / 64;
#pragma unroll
    for (int kk = 0; kk < HP; ++kk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float4 c4 = cf[kk][e >> 1];
            const float cs_x = (e & 1) ? c4.z : c4.x, cs_y = (e & 1) ? c4.w : c4.y;
            const uint32_t w1 = x[kk][e >> 1], w2 = x[kk + HP][e >> 1];
            const float x1 = (e & 1) ? hi_bf16(w1) : lo_bf16(w1);
            const float x2 = (e & 1) ? hi_bf16(w2) : lo_bf16(w2);
            y[kk][e] = (__bf16)(x1 * cs_x - x2 * cs_y);
            y[kk + HP][e] = (__bf16)(x2 * cs_x + x1 * cs_y);
        }
    }
}

typedef __attribute__((address_space(3))) void lds_void;

// The LDS destination of a direct global->LDS load, passed through an empty asm
// so that the compiler cannot tie it to an LDS object: its own wait insertion
// then leaves such loads alone (it would otherwise wait for every outstanding
// load before LDS reads it cannot disambiguate).  Every read of DMA-written
// data is preceded by an explicit vmcnt wait and lds_fence(), and a buffer is
// refilled only after lgkmcnt(0), i.e. after the wave's reads of it are done.
__device__ __forceinline__ lds_void* opaque_lds(unsigned char* p) {
    // wave-uniform by construction; readfirstlane tells the compiler so
    unsigned off = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void*)p);
    asm volatile("" : "+s"(off));
    return (lds_void*)(size_t)off;
}

// The same from an LDS address already converted (lds_u32): the conversion
// of a generic pointer to an LDS address tests it for null, a 64-bit scalar
// compare and select per load when done for every load.
__device__ __forceinline__ uint32_t lds_u32(unsigned char* p) { return (uint32_t)(size_t)(lds_void*)p; }

__device__ __forceinline__ lds_void* opaque_lds(uint32_t a) {
    unsigned off = __builtin_amdgcn_readfirstlane(a);
    asm volatile("" : "+s"(off));
    return (lds_void*)(size_t)off;
}

// Compiler-level memory barrier (no instruction): loads and stores do not move
// across it.
__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, opaque_lds(lds_dst), 16, 0, 0);
}

// The same with the non-temporal cache policy when STREAM (data read once per
// launch and too large to stay cached until the next: the decode walk's K and
// V at large batch).  Its lines leave the L2 early, so the small data every
// block re-reads (the rotation table rows, one per visit) stays resident: the
// decode launch takes about 4.5 us less at the 64-stream 3B shape.  A window
// set that fits in the caches (one stream: the next step reads it again) is
// better served by the default policy, and the chunk kernel gains nothing from
// it (within 0.1 us with K, V or both streaming).
template <bool STREAM>
__device__ __forceinline__ void dma16_policy(const void* src, unsigned char* lds_dst) {
    constexpr int kNonTemporal = 2;   // cache-policy bit NT of the load
    __builtin_amdgcn_global_load_lds(src, opaque_lds(lds_dst), 16, 0, STREAM ? kNonTemporal : 0);
}

// The decode walk's global->LDS loads go through buffer resources (make_rsrc):
// a lane's offsets inside a tile are computed once and each visit adds only
// its tile's scalar byte offset (a global load needs a 64-bit per-lane address
// computed for every load).
template <bool STREAM>
__device__ __forceinline__ void bdma16(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds_dst) {
    constexpr int kNonTemporal = 2;   // cache-policy bit NT of the load
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, opaque_lds(lds_dst), 16, voff, soff, 0, STREAM ? kNonTemporal : 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8): "at most n vector-memory operations outstanding", and
// "no LDS operation outstanding".
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// Waves per decode block: one visit buffer each, two waves per SIMD, so one
// wave's rotation and MFMA work overlaps the other's loads.
constexpr int kDecWaves = 8;

// K part of a visit buffer: chunk (row r, 16-byte column col) of the 32 x D
// tile at chunk position (D/8) r + 8 (col / 8) + ((col % 8) ^ swz(r)).  Each
// DMA instruction then reads 64 / (D/8) consecutive rows (whole cache lines),
// and the MFMA operand reads of eight consecutive lanes (rows tb(n)) fall on
// distinct banks.  The visit's query-rotation row follows the 32 rows.
__device__ __forceinline__ int k_swz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

template <int D>
__device__ __forceinline__ int k_pos(int r, int col) {
    return (D / 8) * r + 8 * (col >> 3) + ((col & 7) ^ k_swz(r));
}

template <int D>
struct DecBuf {
    static constexpr int kK = 2 * (D / 32) * 1024 + 1024;   // K rows + rotation row
    static constexpr int kV = (D / 16) * 1024;
    static constexpr int nK = 2 * (D / 32) + 1;              // DMA instructions per part
    static constexpr int nV = D / 16;
};

// Row `row` of the rotation table (D/2 float2 = 4D bytes) into LDS; lanes past
// the row re-read its last 16 bytes.
template <int D>
__device__ __forceinline__ void dma_table_row(const float2* table, int row, int lane, unsigned char* dst) {
    const int off = 16 * lane < 4 * D ? 16 * lane : 4 * D - 16;
    dma16((const unsigned char*)(table + (int64_t)row * (D / 2)) + off, dst);
}

// The coefficient row staged after the K rows: R(r_q - rho), the query's
// rotation for this visit (R(r_q) when the keys are stored rotated to their
// index).
// The lane's fixed offsets of the decode walk's buffer loads (dec_load_k /
// dec_load_v): K row r = RPI j + lane / (D/8) of a tile, its swizzled
// 16-byte column, for load j; the 8 slots of V dim n of the tile's 8-slot
// block gq; 16 bytes of a table row (lanes past the row re-read its end).
// Load j covers rows RPI j .. RPI j + RPI - 1 (RPI = 4 or 8 rows of 1024 / RPI
// bytes): its rows start 1024 j bytes into the tile, and a row's swizzle
// k_swz(r) takes bits 0-1 from the lane's row rl and bit 2 from (RPI j) >> 3,
// so two per-lane offsets serve every load (fewer registers held across the
// walk).
template <int D>
__device__ __forceinline__ int dec_k_class(int j) {
    return ((64 / (D / 8)) * j >> 3) & 1;
}

template <int D>
__device__ __forceinline__ void dec_lane_offsets(DecodeCtx& c, int lane) {
    constexpr int RPI = 64 / (D / 8);            // rows per instruction
    static_assert(RPI == 4 || RPI == 8, "rows per load");
    const int rl = lane / (D / 8), sl = lane % (D / 8);
#pragma unroll
    for (int cls = 0; cls < 2; ++cls) {
        const int r = rl + 8 * cls;              // a row with the class's swizzle
        const int col = 8 * (sl >> 3) + ((sl & 7) ^ k_swz(r));
        c.koff[cls] = (uint32_t)((rl * D + 8 * col) * 2);
    }
    c.voff = (uint32_t)(((c.gq * D + c.n) * 8) * 2);
    c.toff = (uint32_t)(16 * lane < 4 * D ? 16 * lane : 4 * D - 16);
}

template <int D, bool STREAM>
__device__ __forceinline__ void dec_load_k(const DecodeCtx& c, int k, int lane, uint32_t kbuf) {
    const VisitSrc vs = visit_src(c, k);
    const uint32_t tile_off = (uint32_t)vs.tile * (kTile * D * 2);
#pragma unroll
    for (int j = 0; j < 2 * (D / 32); ++j)
        bdma16<STREAM>(c.kr, c.koff[dec_k_class<D>(j)], tile_off + 1024 * j, kbuf + j * 1024);
    bdma16<false>(c.tr, c.toff, (uint32_t)(c.rq - (c.prerot ? 0 : vs.rho)) * (D * 4), kbuf + 2 * (D / 32) * 1024);
}

template <int D, bool STREAM>
__device__ __forceinline__ void dec_load_v(const DecodeCtx& c, int k, uint32_t vbuf) {
    const VisitSrc vs = visit_src(c, k);
    const uint32_t tile_off = (uint32_t)vs.tile * (kTile * D * 2);
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) bdma16<STREAM>(c.vr, c.voff, tile_off + nb * 256, vbuf + nb * 1024);
}

// A visit's K part copied from LDS into registers: the query-rotation pairs
// R(r_q - rho) and the lane's two K rows (tb0, tb1; dims 8*gq + 32*kk + e), so
// that the buffer can be refilled before the arithmetic starts.  The rows are
// the keys as appended; dec_scores rotates them by R(tb0), R(tb1).
template <int D>
struct DecK {
    float4 qc[D / 64][4];
    u32x4 k0[D / 32], k1[D / 32];
};

template <int D>
__device__ __forceinline__ void dec_read_k(const DecodeCtx& c, const unsigned char* kbuf, DecK<D>& r) {
    constexpr int KK = D / 32;
    lds_coef<D>(kbuf + KK * 2048, c.gq, r.qc);
    const u32x4* kt = (const u32x4*)kbuf;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        r.k0[kk] = kt[k_pos<D>(c.tb0, c.gq + 4 * kk)];
        r.k1[kk] = kt[k_pos<D>(c.tb1, c.gq + 4 * kk)];
    }
}

// Scores of visit k from its K part and the online-softmax update; returns
// this lane's eight probabilities (keys 8*gq .. 8*gq+7, head n) as bf16.
// SEAM: k may be the ring's first visit (only a wave's first visit can be).
// lds_kc: the table rows R(t), t < 32, staged swizzled (lds_coef_t; unused
// when the keys are stored rotated to their index).
template <int D, bool SEAM>
__device__ __forceinline__ bf16x8 dec_scores(const DecodeCtx& c, int k, const DecK<D>& r,
                                             const unsigned char* lds_kc,
                                             const u32x4 (&qraw)[D / 32], const unsigned char* lds_rw,
                                             floatx4 (&o)[D / 16], float& m, float& l) {
    constexpr int KK = D / 32, NB = D / 16;
    const VisitSrc vs = visit_src(c, k);
    const int s0 = vs.s0, rho = vs.rho;
    bf16x8 qb[KK];
    rotate_row<D>(r.qc, qraw, qb);            // query by R(r_q - rho)
    bf16x8 ka[KK], kb[KK];                    // key rows tb0, tb1 by R(tb0), R(tb1)
    if (!c.prerot) {
        float4 cf[D / 64][4];
        lds_coef_t<D>(lds_kc, c.tb0, c.gq, cf);
        rotate_row<D>(cf, r.k0, ka);
        lds_coef_t<D>(lds_kc, c.tb1, c.gq, cf);
        rotate_row<D>(cf, r.k1, kb);
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            ka[kk] = __builtin_bit_cast(bf16x8, r.k0[kk]);
            kb[kk] = __builtin_bit_cast(bf16x8, r.k1[kk]);
        }
    }
    const bool seam = SEAM && (k == 0) && (c.t_o > 0);
    floatx4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        sc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qb[kk], sc0, 0, 0, 0);
        sc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], qb[kk], sc1, 0, 0, 0);
    }
    if (seam && !c.prerot) {
        // the seam visit (wave-uniform): keys behind the oldest slot sit W
        // further on, so they take the query rotated by R(r_q - rho - W)
        // (composed pair by pair from R(r_q - rho) and the R(W) row in LDS)
        bf16x8 qbw[KK];
        {
            constexpr int HP = D / 64;
            const float4* wrow = (const float4*)lds_rw + 4 * c.gq;
#pragma unroll
            for (int kk = 0; kk < HP; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float4 a4 = r.qc[kk][e >> 1], w4 = wrow[16 * kk + (e >> 1)];
                    const float ax = (e & 1) ? a4.z : a4.x, ay = (e & 1) ? a4.w : a4.y;
                    const float wx = (e & 1) ? w4.z : w4.x, wy = (e & 1) ? w4.w : w4.y;
                    const float cx = ax * wx + ay * wy, cy = ay * wx - ax * wy;
                    const uint32_t u1 = qraw[kk][e >> 1], u2 = qraw[kk + HP][e >> 1];
                    const float x1 = (e & 1) ? hi_bf16(u1) : lo_bf16(u1);
                    const float x2 = (e & 1) ? hi_bf16(u2) : lo_bf16(u2);
                    qbw[kk][e] = (__bf16)(x1 * cx - x2 * cy);
                    qbw[kk + HP][e] = (__bf16)(x2 * cx + x1 * cy);
                }
        }
        floatx4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            w0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qbw[kk], w0, 0, 0, 0);
            w1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], qbw[kk], w1, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {                 // element j: keys 8 gq + j and 8 gq + 4 + j
            sc0[j] = 8 * c.gq + j < c.t_o ? w0[j] : sc0[j];
            sc1[j] = 8 * c.gq + 4 + j < c.t_o ? w1[j] : sc1[j];
        }
    }
    const float sl = c.scale_log2;
    float s[8] = {sc0[0] * sl, sc0[1] * sl, sc0[2] * sl, sc0[3] * sl,
                  sc1[0] * sl, sc1[1] * sl, sc1[2] * sl, sc1[3] * sl};
    const bool full = vs.pre ? (s0 + kTile <= c.F) : ((k != 0) && (rho + kTile <= c.L) && (s0 + kTile <= c.W));
    if (!full) {
        // branch-free: key index of each score, then a select (a prefix tile:
        // its live tokens, all before the query)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tt = 8 * c.gq + e;
            const int rr = rho + tt + ((seam & (tt < c.t_o)) ? c.W : 0);
            const bool ok_ring = (rr >= 0) & (rr < c.L) & (s0 + tt < c.W);
            const bool ok_pre = s0 + tt < c.F;
            const bool ok = vs.pre ? ok_pre : ok_ring;
            s[e] = ok ? s[e] : -INFINITY;
        }
    }
    float mx = s[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
    mx = max_rows4(mx);
    // lazy rescale: keep the running max unless a score exceeds it by 2^8; the
    // branch is taken by the whole wave when any column needs it (the others
    // multiply by exactly 1)
    const bool grow = mx > m + 8.f;
    if (__any(grow)) {
        const float mn = grow ? mx : m;
        const float alpha = fast_exp2(m - mn);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < NB; ++i) o[i] *= alpha;
        m = mn;
    }
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float pe = fast_exp2(s[e] - m);
        l += pe;
        pb[e] = (__bf16)pe;
    }
    return pb;
}

template <int D>
__device__ __forceinline__ void dec_read_v(const unsigned char* vbuf, int lane, u32x4 (&v)[D / 16]) {
    const u32x4* lb = (const u32x4*)vbuf + lane;       // each lane reads the 16 bytes it loaded
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) v[nb] = lb[nb * 64];
}

template <int D>
__device__ __forceinline__ void dec_pv(const u32x4 (&v)[D / 16], bf16x8 pb, floatx4 (&o)[D / 16]) {
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v[nb]), pb, o[nb], 0, 0, 0);
}

// The new token (fused append) written into the LDS copy of its tile: K row t
// (16-byte chunk `lane` of dims 8*lane ..) and element t % 8 of the
// transposed V chunks of block t / 8.
template <int D>
__device__ __forceinline__ void patch_k(unsigned char* kbuf, int t, int lane, u32x4 tk) {
    if (lane < D / 8) *(u32x4*)(kbuf + 16 * k_pos<D>(t, lane)) = tk;
}

template <int D>
__device__ __forceinline__ void patch_v(unsigned char* vbuf, int t, int lane, u32x4 tv) {
    if (lane < D / 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int d = 8 * lane + u;
            const uint32_t w = tv[u >> 1];
            *(uint16_t*)(vbuf + (d >> 4) * 1024 + 16 * ((d & 15) + 16 * (t >> 3)) + 2 * (t & 7)) =
                (uint16_t)((u & 1) ? (w >> 16) : (w & 0xffffu));
        }
    }
}

// A normalized split partial (o = O / l, lse = m + log2 l, base 2) packed in
// 64 bits: lse in the high word, o in the low word.  A NaN lse is written as
// the canonical quiet NaN, so a packed partial is never kSlotEmpty (all ones).
__device__ __forceinline__ uint64_t pack_partial(float o, float lse) {
    uint32_t hi = __float_as_uint(lse);
    if (hi == 0xffffffffu) hi = 0x7fc00000u;
    return ((uint64_t)hi << 32) | __float_as_uint(o);
}

// Merge of two packed partials, a first: weights 2^(lse - max); two empty
// partials (lse = -inf) stay empty.
__device__ __forceinline__ uint64_t merge_partials(uint64_t a, uint64_t b) {
    const float la = __uint_as_float((uint32_t)(a >> 32)), lb = __uint_as_float((uint32_t)(b >> 32));
    const float mx = fmaxf(la, lb);
    if (mx == -INFINITY) return a;
    const float wa = fast_exp2(la - mx), wb = fast_exp2(lb - mx);
    const float sw = wa + wb;
    const float o = (__uint_as_float((uint32_t)a) * wa + __uint_as_float((uint32_t)b) * wb) * __builtin_amdgcn_rcpf(sw);
    return pack_partial(o, mx + __builtin_amdgcn_logf(sw));
}

template <int D, bool PREROT, bool PRE, bool STREAM>
__global__ __launch_bounds__(64 * kDecWaves, 1) void decode_mfma(Geometry g, int layer, StreamBatch st,
                                                                const uint16_t* __restrict__ q,
                                                                uint16_t* __restrict__ out, int n_split,
                                                                const uint16_t* __restrict__ k_new,
                                                                const uint16_t* __restrict__ v_new) {
    constexpr int KK = D / 32, NB = D / 16, NWV = kDecWaves;
    using B = DecBuf<D>;
    // per wave one visit buffer, a K part and a V part (two LDS objects); then
    // the block's query rows, R(W) row, new token and the R(t) rows t < 32
    __shared__ __align__(16) unsigned char lds_k[NWV * B::kK];
    __shared__ __align__(16) unsigned char lds_v[NWV * B::kV];
    __shared__ __align__(16) unsigned char lds_q[4096];
    __shared__ __align__(16) unsigned char lds_rw[1024];
    __shared__ __align__(16) unsigned char lds_tok[1024];
    __shared__ __align__(16) unsigned char lds_kc[kTile * D * 4];
    __shared__ float red_ml[NWV][16][2];
    // rows padded by 4 floats: the float4 writes of a column group's 16 lanes
    // (one row each) then spread over the banks
    constexpr int kRow = D + 4;
    static_assert(NWV * 16 * kRow * 4 <= NWV * B::kK, "merge buffer does not fit");
    float (*red_o)[16][kRow] = (float (*)[16][kRow])lds_k;   // after the walk

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const int bi = blockIdx.z, kh = blockIdx.y, split = blockIdx.x;
    const int b = st.b0 + bi, G = g.group, W = g.window;
    const bool fused = k_new != nullptr;
    unsigned char* ka = lds_k + wave * B::kK;
    unsigned char* va = lds_v + wave * B::kV;
    const uint32_t ka_u = lds_u32(ka), va_u = lds_u32(va);

    // window after the (optional) append of one token
    const int s_prev = st.next_slot[bi];
    const int L = fused ? min(st.length[bi] + 1, W) : st.length[bi];
    const int next_slot = fused ? wrap_slot(s_prev + 1, W) : s_prev;
    DecodeCtx c;
    c.L = L;
    c.W = W;
    c.oldest = next_slot - L < 0 ? next_slot - L + W : next_slot - L;
    c.rq = L - 1;
    c.n_tiles = g.w_pad / kTile;
    c.p0t = c.oldest / kTile;
    c.t_o = c.oldest - c.p0t * kTile;
    c.tb0 = 8 * (n >> 2) + (n & 3);
    c.tb1 = c.tb0 + 4;
    c.gq = gq;
    c.n = n;
    c.scale_log2 = g.scale_log2;
    c.prerot = PREROT;   // compile-time constants: the method's instance carries none of the variant
    c.pre_on = PRE;      // and, without a prefix in the batch, none of the prefix walk
    c.table = g.table;
    const int64_t pair = pair_index(g, layer, b, kh);
    c.kp = (const uint16_t*)g.k_ring + pair * g.pair_slots * D;
    c.vp = (const uint16_t*)g.v_ring + pair * g.pair_slots * D;
    c.kr = make_rsrc(c.kp, (uint32_t)g.pair_slots * D * 2);
    c.vr = make_rsrc(c.vp, (uint32_t)g.pair_slots * D * 2);
    c.tr = make_rsrc(g.table, (uint32_t)(g.window + g.f_pad + kTablePad) * D * 4);
    dec_lane_offsets<D>(c, lane);
    int n_visit;
    {
        int last = c.oldest + L - 1;
        if (last < W) {
            n_visit = last / kTile - c.p0t + 1;
        } else {
            last -= W;
            n_visit = c.n_tiles - c.p0t + last / kTile + 1;
            if (n_visit > c.n_tiles) n_visit = c.n_tiles;
        }
    }
    // then the pinned prefix's tiles
    c.F = PRE ? st.prefix[bi] : 0;
    c.n_roll = n_visit;
    n_visit += (c.F + kTile - 1) / kTile;
    const int per = (n_visit + n_split - 1) / n_split;
    const int k0 = split * per, k1 = min(n_visit, k0 + per);

    // Table rows 0 .. 31 (R(t), t < 32) into lds_kc, swizzled (see
    // lds_coef_t), an equal share per wave; the oldest loads of the kernel, so
    // the prologue's wait covers them
    if (!PREROT) {
        constexpr int kChunks = D / 4;                  // 16-byte chunks per row
        constexpr int kInstr = kTile * kChunks / 64;    // loads for 32 rows
        static_assert(kInstr % NWV == 0, "table rows are not split evenly");
        const uint32_t kc_u = lds_u32(lds_kc);
#pragma unroll
        for (int u = 0; u < kInstr / NWV; ++u) {
            const int j = wave * (kInstr / NWV) + u;
            const int p = j * 64 + lane;                 // destination chunk
            const int row = p / kChunks, col = p % kChunks;
            bdma16<false>(c.tr, (uint32_t)(16 * (col ^ k_swz(row))), (uint32_t)row * (D * 4), kc_u + 1024 * j);
        }
    }

    // Fused append: the wave whose visits include the new token's tile (visit
    // k_tok) loads the token into LDS with its prologue, patches it into its
    // LDS copy of that tile once the tile has landed, and writes it into the
    // ring slot after the walk, so nothing waits for a store (no other wave or
    // block reads that slot in this call).
    int k_tok = -1;
    const int t_tok = s_prev & (kTile - 1);
    if (fused) {
        int kv = s_prev / kTile - c.p0t;
        if (kv < 0) kv += c.n_tiles;
        if (kv >= k0 && kv < k1 && (kv - k0) % NWV == wave) {
            // at most one wave per block: the token's K row to lds_tok[0, 2D),
            // its V row to [2D, 4D) (other lanes re-read the K row's start)
            k_tok = kv;
            const int64_t src = ((int64_t)bi * g.hkv + kh) * D;
            const void* from = lane < D / 8   ? (const void*)(k_new + src + 8 * lane)
                             : lane < D / 4   ? (const void*)(v_new + src + 8 * (lane - D / 8))
                                              : (const void*)(k_new + src);
            dma16(from, lds_tok + 16 * lane);
        }
    }

    // Prologue, every load a direct global->LDS load (so the explicit wait
    // counts are exact): a quarter of the query block each for waves 0 .. 3
    // (clamped to it), the R(W) row (wave 0), ...
    int k = k0 + wave;
    {
        const int qbytes = G * D * 2;
        int qo = wave * 1024 + 16 * lane;
        qo = qo < qbytes ? qo : qbytes - 16;
        if (wave < 4) dma16((const unsigned char*)(q + ((int64_t)bi * g.hq + kh * G) * D) + qo, lds_q + wave * 1024);
        if (wave == 0) dma_table_row<D>(g.table, W, lane, lds_rw);
    }
    // then K(k) and V(k) of the wave's first visit (if it exists), and a wait
    // for everything up to K(k)
    if (k < k1) {
        dec_load_k<D, STREAM>(c, k, lane, ka_u);
        dec_load_v<D, STREAM>(c, k, va_u);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(B::nV));
    } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __builtin_amdgcn_s_barrier();                                    // ... and every other wave's
    lds_fence();

    // the query stays as bf16 bits (the softmax scale is applied to the
    // scores), held in registers; the prefix instance, short of registers,
    // re-reads it from LDS at every visit instead (held there it spilled, and
    // the spill reloads' waits drained the walk's loads)
    const unsigned char* qrow = lds_q + (n < G ? n : 0) * D * 2 + 16 * gq;
    u32x4 qraw[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qraw[kk] = *(const u32x4*)(qrow + 64 * kk);

    floatx4 o[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = kNegBig, l = 0.f;

    // Visits k0 + wave, + NWV, ... through the wave's one buffer.  Per visit:
    // wait for its K part, copy it to registers, refill the K part with the
    // wave's next visit (if there is one), compute the scores; then the same
    // for the V part and PV.  The loads in flight after K(k) are V(k); after
    // V(k), K(k + NWV) if it was issued.  The two waves sharing a SIMD overlap
    // one's arithmetic with the other's loads.
    auto wait_k = [&]() {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(B::nV));
        __builtin_amdgcn_sched_barrier(0);
        lds_fence();
    };
    auto wait_v = [&](int kk) {
        if (kk + NWV < k1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(B::nK));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_sched_barrier(0);
        lds_fence();
    };
    bool first = true;
    while (k < k1) {
        DecK<D> rk;
        u32x4 rv[NB];
        wait_k();
        if (k == k_tok) patch_k<D>(ka, t_tok, lane, ((const u32x4*)lds_tok)[lane & (D / 8 - 1)]);
        dec_read_k<D>(c, ka, rk);
        __builtin_amdgcn_s_waitcnt(kLgkm0);                                 // copied out of ka
        if (k + NWV < k1) dec_load_k<D, STREAM>(c, k + NWV, lane, ka_u);
        if (PRE) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) qraw[kk] = *(const u32x4*)(qrow + 64 * kk);
        }
        bf16x8 pb = first ? dec_scores<D, true>(c, k, rk, lds_kc, qraw, lds_rw, o, m, l)
                          : dec_scores<D, false>(c, k, rk, lds_kc, qraw, lds_rw, o, m, l);
        first = false;
        wait_v(k);
        if (k == k_tok) patch_v<D>(va, t_tok, lane, ((const u32x4*)lds_tok)[D / 8 + (lane & (D / 8 - 1))]);
        dec_read_v<D>(va, lane, rv);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        if (k + NWV < k1) dec_load_v<D, STREAM>(c, k + NWV, va_u);
        dec_pv<D>(rv, pb, o);
        k += NWV;
    }
    __builtin_amdgcn_s_waitcnt(0);   // every load has landed before the LDS is reused
    lds_fence();

    if (k_tok >= 0 && lane < D / 8)     // the new token into its ring slot, for later calls
        write_token_vals<2>(g, pair, s_prev, lane, ((const u32x4*)lds_tok)[lane], ((const u32x4*)lds_tok)[D / 8 + lane]);

    if (fused && kh == 0 && split == 0 && tid == 0) {   // record of the new state
        DevState ns;
        ns.next_pos = st.next_pos[bi] + 1;
        ns.length = L;
        ns.next_slot = next_slot;
        g.state[(int64_t)layer * g.n_streams + b] = ns;
    }

    // Across the block's waves: each wave rescales its {l, O} to the block's
    // running max before writing them, so that the per-element merge is a sum.
    // The first barrier also means every wave is done with its visit buffers,
    // which red_o overlays.
    l = sum_rows4(l);
    if (n < G && gq == 0) red_ml[wave][n][0] = m;
    __syncthreads();
    {
        const int hn = n < G ? n : 0;
        float mb = red_ml[0][hn][0];
#pragma unroll
        for (int w = 1; w < NWV; ++w) mb = fmaxf(mb, red_ml[w][hn][0]);
        const float f = fast_exp2(m - mb);
        if (n < G) {
            if (gq == 0) red_ml[wave][n][1] = l * f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                *(float4*)&red_o[wave][n][16 * nb + 4 * gq] =
                    float4{o[nb][0] * f, o[nb][1] * f, o[nb][2] * f, o[nb][3] * f};
        }
    }
    __syncthreads();

    // The block's partial {m, l, O} for each (head, dim) this thread owns.
    //
    // The splits of one (stream, KV head) merge per output element in a fixed
    // binary tree: at each level the nodes 2m and 2m + 1 (splits at the first
    // level; the launcher passes a power of two, so every node has its partner)
    // meet in an exchange slot that holds kSlotEmpty between calls.  Each carrier swaps in its node's
    // normalized partial (O / l, m + log2 l) with one 64-bit atomic exchange;
    // the one that gets its partner's partial back (it came second) merges the
    // two (node 2m always as the first operand), empties the slot and carries
    // the result up; the one that gets kSlotEmpty back is done with that
    // element.  Whoever carries it, a node's value is the same function of its
    // children's, so results are the same run to run.  One round trip per
    // level; two splits (the usual case) take one level and no block-wide
    // count.
    constexpr int kThr = 64 * NWV;
    constexpr int kPer = (kMaxGroupMfma * D + kThr - 1) / kThr;
    float p_num[kPer], p_den[kPer], p_m[kPer];
    // elements of this thread: the same count across a wave (G * D is a
    // multiple of 64), so the loops below branch uniformly
    const int n_mine = __builtin_amdgcn_readfirstlane((G * D - 64 * wave + kThr - 1) / kThr);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (i >= n_mine) break;
        const int idx = tid + kThr * i;
        const int h = idx / D, d = idx - h * D;
        float mm = red_ml[0][h][0], num = red_o[0][h][d], den = red_ml[0][h][1];
#pragma unroll
        for (int w = 1; w < NWV; ++w) {
            mm = fmaxf(mm, red_ml[w][h][0]);
            num += red_o[w][h][d];
            den += red_ml[w][h][1];
        }
        p_num[i] = num;
        p_den[i] = den;
        p_m[i] = mm;
    }
    auto out_at = [&](int idx) -> uint16_t& { return out[((int64_t)bi * g.hq + kh * G) * D + idx]; };
    if (n_split == 1) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (i >= n_mine) break;
            out_at(tid + kThr * i) = f32_to_bf16_bits(p_num[i] / p_den[i]);
        }
        return;
    }
    // slot rows node-major, [node][stream][kv head][head][D]: the first node's
    // rows of all pairs (all that two splits use) are contiguous
    const int64_t node_stride = (int64_t)g.n_streams * g.hkv * kMaxGroupMfma * D;
    uint64_t* const slots = g.part_x + ((int64_t)bi * g.hkv + kh) * kMaxGroupMfma * D + tid;
    if (n_split == 2) {
        // one level: the same exchange written out (every exchange issued
        // before any result is needed, the merge and the output store
        // straight after)
        uint64_t x_mine[kPer], x_old[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (i >= n_mine) break;
            const bool live = p_den[i] > 0.f;
            const float on = live ? p_num[i] * __builtin_amdgcn_rcpf(p_den[i]) : 0.f;
            x_mine[i] = pack_partial(on, live ? p_m[i] + __builtin_amdgcn_logf(p_den[i]) : -INFINITY);
            x_old[i] = __hip_atomic_exchange(slots + kThr * i, x_mine[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (i >= n_mine) break;
            if (x_old[i] == kSlotEmpty) continue;             // the other split merges it
            const uint64_t a = split == 0 ? x_mine[i] : x_old[i], c1 = split == 0 ? x_old[i] : x_mine[i];
            const float la = __uint_as_float((uint32_t)(a >> 32)), lb = __uint_as_float((uint32_t)(c1 >> 32));
            const float mx = fmaxf(la, lb);
            const float wa = fast_exp2(la - mx), wb = fast_exp2(lb - mx);
            const float r = (__uint_as_float((uint32_t)a) * wa + __uint_as_float((uint32_t)c1) * wb) *
                            __builtin_amdgcn_rcpf(wa + wb);
            out_at(tid + kThr * i) = f32_to_bf16_bits(r);
            __hip_atomic_store(slots + kThr * i, kSlotEmpty, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    // normalized partials; an empty split (short window) has den = 0 and
    // enters as (0, -inf), weight 0 in every merge
    uint64_t xv[kPer];
    bool carry[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) carry[i] = i < n_mine;   // every entry set: the loops below test all kPer
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (i >= n_mine) break;
        const bool live = p_den[i] > 0.f;             // then den >= 1 (the max term is 1)
        const float on = live ? p_num[i] * __builtin_amdgcn_rcpf(p_den[i]) : 0.f;
        xv[i] = pack_partial(on, live ? p_m[i] + __builtin_amdgcn_logf(p_den[i]) : -INFINITY);
    }
    int node = split, width = n_split, base = 0;   // wave-uniform
    while (width > 1) {
        {
            uint64_t* sl = slots + (base + (node >> 1)) * node_stride;
            uint64_t old[kPer];
            // every exchange of the level issued before any result is needed
#pragma unroll
            for (int i = 0; i < kPer; ++i)
                if (carry[i]) old[i] = __hip_atomic_exchange(sl + kThr * i, xv[i], __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                if (!carry[i]) continue;
                if (old[i] == kSlotEmpty) {            // the partner carries this element on
                    carry[i] = false;
                    continue;
                }
                xv[i] = (node & 1) ? merge_partials(old[i], xv[i]) : merge_partials(xv[i], old[i]);
                __hip_atomic_store(sl + kThr * i, kSlotEmpty, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        base += width >> 1;
        node >>= 1;
        width >>= 1;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (carry[i]) out_at(tid + kThr * i) = f32_to_bf16_bits(__uint_as_float((uint32_t)xv[i]));
}

// ---------------------------------------------------------- pipelined chunk --
// bf16 attention for C new positions per stream, one block per (stream, KV
// head, split, row group of up to 128 of the C x G query rows; row = c*G + hg;
// more than one row group re-reads the window), in WG groups
// of 4 waves that take alternate visits of the split and merge at the end.
// Within a group wave w owns the query column blocks w, w + 4 (16 rows each)
// for the whole walk, and each wave issues a quarter of every visit's loads
// (LDS DMA).
// Rotation: each query row is rotated once, by its own re-based index
// r_q(c) = L - C + c; key t of a visit (stored as appended) by R(rho + t),
// composed in float32 from R(rho), the table row staged with the visit, and
// R(t), which the lane that rotates key t keeps in registers.  On the first
// visit rho = -t_o (R(t_o) conjugated), and the window's newest keys that share
// the oldest key's tile (t < t_o, index t - t_o + W) get R(W) composed on top.  Query c sees
// keys with index <= r_q(c): causal inside the chunk, the whole older window
// before it.  With several splits each block writes its rows' partials
// {m, l, O} and combine_kernel, launched next, merges them (a chip-wide merge
// instead of one block reading every split's partials).
//
// Visit rings of one wave group: K parts (the 32 raw K rows and the visit's
// R(rho) row) and V parts in separate rings, and two rotated-K tiles.  At step
// s a group rotates the keys of its visit s + 1 into one tile while it runs
// QK^T, the online softmax and PV of visit s on the other, so a step has one
// barrier and the rotation's VALU work overlaps the MFMAs.  K(v) is loaded
// three steps before its rotation, V(v) two steps before its PV.
template <int D>
struct PipeBuf {
    static constexpr int kK = kTile * D * 2;           // raw K rows, row r at r * 2D bytes
    static constexpr int kC = D * 4;                   // the R(rho) row (D/2 float2)
    static constexpr int kKC = kK + kC;                 // one K slot
    static constexpr int kV = kTile * D * 2;           // V chunks, as in the decode buffers
    static constexpr int kT = kTile * D * 2;           // a rotated-K tile (XOR-swizzled rows)
    static constexpr int dK = 3, dV = 3;               // ring depths
    static constexpr int kGroup = dK * kKC + dV * kV + 2 * kT;
    static constexpr int nK = 2 * (D / 32) / 4 + 1;    // DMA instructions per wave: K rows + row quarter
    static constexpr int nV = (D / 16) / 4;
};

template <int D, int NW, int WG, bool PRE>
__global__ __launch_bounds__(256 * WG, 1) void chunk_pipe(Geometry g, int layer, StreamBatch st, int C,
                                                     const uint16_t* __restrict__ q,
                                                     uint16_t* __restrict__ out, int n_split,
                                                     const uint16_t* __restrict__ k_new,
                                                     const uint16_t* __restrict__ v_new) {
    constexpr int KK = D / 32, NB = D / 16, HP = D / 64;
    constexpr int P = D / 16;                          // rotation pairs per lane (8 lanes per key)
    using PB = PipeBuf<D>;
    __shared__ __align__(16) unsigned char lds_all[WG * PB::kGroup];
    __shared__ __align__(16) unsigned char lds_rw[1024];
    __shared__ __align__(16) unsigned char lds_qc[8 * 1024];        // R(L - C + c) rows, c < C
    static_assert(kMaxPartialQ * D * 4 <= 8 * 1024, "query rotation rows do not fit");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_b = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wg = wave_b >> 2, wave = wave_b & 3;      // wave group, wave within the group
    unsigned char* gb = lds_all + wg * PB::kGroup;
    unsigned char* const ring_k = gb;                                   // dK slots
    unsigned char* const ring_v = gb + PB::dK * PB::kKC;                // dV slots
    unsigned char* const tiles = ring_v + PB::dV * PB::kV;              // 2 rotated tiles
    const int n = lane & 15, gq = lane >> 4;
    const int bi = blockIdx.z, kh = blockIdx.y;
    const int split = blockIdx.x % n_split, row0 = 128 * (blockIdx.x / n_split);
    const int b = st.b0 + bi, G = g.group, W = g.window;
    const int rows = C * G;                            // rows of this block: row0 + 16 (wave + 4w) + n

    // window after the (optional) append of the C new tokens: with k_new the
    // state in the arguments is the state before it
    const bool fused = k_new != nullptr;
    const int s_prev = st.next_slot[bi];
    const int L = fused ? min(st.length[bi] + C, W) : st.length[bi];
    const int next_slot = fused ? wrap_slot(s_prev + C, W) : s_prev;
    DecodeCtx c;
    c.L = L;
    c.W = W;
    c.oldest = next_slot - L < 0 ? next_slot - L + W : next_slot - L;
    c.rq = L - C;                      // index of the chunk's first query
    c.n_tiles = g.w_pad / kTile;
    c.p0t = c.oldest / kTile;
    c.t_o = c.oldest - c.p0t * kTile;
    c.tb0 = 8 * (n >> 2) + (n & 3);
    c.tb1 = c.tb0 + 4;
    c.gq = gq;
    c.n = n;
    c.scale_log2 = g.scale_log2;
    c.prerot = 0;
    c.pre_on = PRE;
    c.table = g.table;
    const int64_t pair = pair_index(g, layer, b, kh);
    c.kp = (const uint16_t*)g.k_ring + pair * g.pair_slots * D;
    c.vp = (const uint16_t*)g.v_ring + pair * g.pair_slots * D;
    c.kr = make_rsrc(c.kp, (uint32_t)g.pair_slots * D * 2);
    c.vr = make_rsrc(c.vp, (uint32_t)g.pair_slots * D * 2);
    c.tr = make_rsrc(g.table, (uint32_t)(g.window + g.f_pad + kTablePad) * D * 4);
    int n_visit;
    {
        int last = c.oldest + L - 1;
        if (last < W) {
            n_visit = last / kTile - c.p0t + 1;
        } else {
            last -= W;
            n_visit = c.n_tiles - c.p0t + last / kTile + 1;
            if (n_visit > c.n_tiles) n_visit = c.n_tiles;
        }
    }
    // then the pinned prefix's tiles
    c.F = PRE ? st.prefix[bi] : 0;
    c.n_roll = n_visit;
    n_visit += (c.F + kTile - 1) / kTile;
    const int per = (n_visit + n_split - 1) / n_split;
    const int k0 = split * per, k1 = min(n_visit, k0 + per);
    // group wg takes visits k0 + wg, k0 + wg + WG, ...: its local visit v is
    // kvis(v); every wave of the block runs n_steps steps (one barrier each)
    const int n_mine = k0 + wg < k1 ? (k1 - k0 - wg + WG - 1) / WG : 0;
    const int n_steps = (k1 - k0 + WG - 1) / WG;
    auto kvis = [&](int v) { return k0 + wg + WG * v; };

    // this wave's quarter of local visit v's K part (rows + a quarter of the
    // R(rho) row, |rho| for the first visit) and of its V part
    // (a v past the group's visits loads the pair's first tile instead, which
    // is always in range; its slot is never read)
    // (buffer loads: the lane's offset inside a tile is fixed, the tile's
    // offset is scalar; LDS slots as 32-bit addresses, converted once)
    const uint32_t ring_k_u = lds_u32(ring_k), ring_v_u = lds_u32(ring_v);
    const uint32_t k_lane = 16 * lane;
    constexpr int q4 = PB::kC / 4;                      // bytes of the R(rho) row per wave
    // staged chunk p = 8 i + c of the R(rho) row holds chunk (P/2) c + i of the table row
    const int row_p = wave * (q4 / 16) + (lane & (q4 / 16 - 1));
    const uint32_t row_lane = 16 * ((P / 2) * (row_p & 7) + (row_p >> 3));
    const uint32_t v_lane = (uint32_t)((gq * D + n) * 16);
    auto issue_k = [&](int v, uint32_t slot) {
        const int kv = v < n_mine ? kvis(v) : 0;
        const VisitSrc vs = visit_src(c, kv);
        const uint32_t tile_off = (uint32_t)vs.tile * (kTile * D * 2);
#pragma unroll
        for (int u = 0; u < PB::nK - 1; ++u) {
            const int j = wave * (PB::nK - 1) + u;
            bdma16<false>(c.kr, k_lane, tile_off + j * 1024, slot + j * 1024);
        }
        const int rho = vs.rho;
        if (lane < q4 / 16)
            bdma16<false>(c.tr, row_lane, (uint32_t)(rho < 0 ? -rho : rho) * (D * 4), slot + PB::kK + wave * q4);
    };
    auto issue_v = [&](int v, uint32_t slot) {
        const VisitSrc vs = visit_src(c, v < n_mine ? kvis(v) : 0);
        const uint32_t tile_off = (uint32_t)vs.tile * (kTile * D * 2);
#pragma unroll
        for (int u = 0; u < PB::nV; ++u) {
            const int nb = wave * PB::nV + u;
            bdma16<false>(c.vr, v_lane, tile_off + nb * 256, slot + nb * 1024);
        }
    };

    // Prologue: register loads (query rows), R(W) into LDS (wave 0), the C
    // consecutive table rows of the queries' rotations into LDS (1 KiB per
    // wave, clamped to them), then K(0), K(1), V(0), issued even where those
    // visits do not exist (then they re-read an in-range tile), so that the
    // first wait below is unconditional.
    const int kr_t = 8 * wave + (lane >> 3);           // key offset this lane rotates
    const int kr_i = P * (lane & 7);                   // its first pair index
    // The staged R(rho) row: lane group c = lane & 7 needs the P/2 16-byte
    // chunks (P/2) c + i of the table row; they are staged at 8 i + c, so the
    // eight groups' reads of one i are consecutive chunks (no bank conflict)
    // at compile-time offsets from the group's base.
    // R(kr_t) for those pairs, for the whole walk (table row kr_t < 32)
    float2 rt[P];
#pragma unroll
    for (int i = 0; i < P; ++i) rt[i] = g.table[(int64_t)kr_t * (D / 2) + kr_i + i];
    u32x4 qr[NW][KK];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        int row = row0 + 16 * (wave + 4 * w) + n;
        if (row >= rows) row = 0;
        const int cc = row / G, h = kh * G + (row - cc * G);
        const uint16_t* qp = q + (((int64_t)bi * C + cc) * g.hq + h) * D + 8 * gq;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qr[w][kk] = *(const u32x4*)(qp + 32 * kk);
    }
    if (wave_b == 0) dma_table_row<D>(g.table, W, lane, lds_rw);
    {
        const int qcb = C * D * 4;
        int off = wave_b * 1024 + 16 * lane;
        off = off < qcb ? off : qcb - 16;
        dma16((const unsigned char*)(g.table + (int64_t)c.rq * (D / 2)) + off, lds_qc + wave_b * 1024);
    }
    // Fused append (one row group): the new tokens of this (stream, KV head)
    // whose tiles are among this block's visits are copied into their ring
    // slots, as append_kernel writes them.  No other block reads those tiles
    // in this call.  The stores must be in the L2 before any wave loads one of
    // those tiles.  When none of them is among the first loads issued below
    // (visits k0 .. k0 + 2 WG - 1), the stores overlap those loads: step -1
    // waits for everything (vmcnt 0) before its barrier, and every later load
    // is issued after that barrier; otherwise the block waits for the stores
    // here (and for the query and table loads above, issued first so that
    // their latency overlaps) before its first K/V load.
    if (fused) {
        auto visit_of = [&](int slot) {
            const int v = slot / kTile - c.p0t;
            return v < 0 ? v + c.n_tiles : v;
        };
        bool mine = false, early = false;               // block-uniform
        for (int j = 0; j < C; ++j) {
            const int v = visit_of(wrap_slot(s_prev + j, W));
            mine = mine || (v >= k0 && v < k1);
            early = early || (v >= k0 && v < k1 && v < k0 + 2 * WG);
        }
        if (mine) {
            constexpr int chunks = D / 8;              // 16-byte chunks of a bf16 row
            for (int t = tid; t < C * chunks; t += 256 * WG) {
                const int j = t / chunks, cc = t - j * chunks;
                const int slot = wrap_slot(s_prev + j, W);
                const int v = visit_of(slot);
                if (v >= k0 && v < k1) {
                    const int64_t src = (((int64_t)bi * C + j) * g.hkv + kh) * D * 2;
                    write_token_chunk<2>(g, pair, slot, cc, (const uint8_t*)k_new + src,
                                         (const uint8_t*)v_new + src);
                }
            }
            if (early) {
                __builtin_amdgcn_s_waitcnt(0);         // the tokens are in the L2 ...
                __syncthreads();                       // ... before any wave loads a tile
            }
        }
        if (kh == 0 && split == 0 && tid == 0) {      // record of the new state
            DevState ns;
            ns.next_pos = st.next_pos[bi] + C;
            ns.length = L;
            ns.next_slot = next_slot;
            g.state[(int64_t)layer * g.n_streams + b] = ns;
        }
    }

    issue_k(0, ring_k_u);
    issue_k(1, ring_k_u + PB::kKC);
    issue_v(0, ring_v_u);

    // column blocks with at least one real row (wave-uniform)
    const bool act0 = row0 + 16 * wave < rows, act1 = NW > 1 && row0 + 16 * (wave + 4) < rows;

    floatx4 o[NW][NB];
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int i = 0; i < NB; ++i) o[w][i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m[NW], l[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        m[w] = kNegBig;
        l[w] = 0.f;
    }
    const int r_last = L - 1;

    // Rotates key kr_t of local visit v (pairs kr_i .. kr_i + P - 1) from its K
    // slot into a rotated tile, by R(rho + kr_t): the visit's staged row R(rho),
    // conjugated where rho < 0 (the ring's first visit, rho = -t_o, and prefix
    // visits; on the first visit keys before the oldest slot, the window's
    // newest, get R(W) on top), composed with the lane's R(kr_t).  The key is
    // rounded to bf16 once, as the MFMA operand.
    auto rotate = [&](const unsigned char* kslot, unsigned char* tile, bool first, bool seam) {
        const float4* brow = (const float4*)(kslot + PB::kK) + (lane & 7);
        auto br = [&](int i2) { return brow[8 * i2]; };
        const unsigned char* kraw = kslot + kr_t * D * 2;
        uint32_t x1w[P / 2], x2w[P / 2];
        if constexpr (P == 8) {
            const u32x4 a1 = *(const u32x4*)(kraw + 2 * kr_i), a2 = *(const u32x4*)(kraw + 2 * (kr_i + D / 2));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x1w[i] = a1[i];
                x2w[i] = a2[i];
            }
        } else {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 a1 = *(const u32x2*)(kraw + 2 * kr_i), a2 = *(const u32x2*)(kraw + 2 * (kr_i + D / 2));
            x1w[0] = a1[0];
            x1w[1] = a1[1];
            x2w[0] = a2[0];
            x2w[1] = a2[1];
        }
        float2 cf[P];
#pragma unroll
        for (int i2 = 0; i2 < P / 2; ++i2) {
            const float4 b4 = br(i2);
            cf[2 * i2] = float2{b4.x, b4.y};
            cf[2 * i2 + 1] = float2{b4.z, b4.w};
        }
        if (first) {                                   // wave-uniform: rho < 0
            const bool wrap = seam && kr_t < c.t_o;    // index kr_t - t_o + W: R(W) on top
            const float4* wr = (const float4*)lds_rw + kr_i / 2;
#pragma unroll
            for (int i2 = 0; i2 < P / 2; ++i2) {
                const float4 b4 = br(i2), w4 = wr[i2];
                const float2 a2[2] = {float2{b4.x, -b4.y}, float2{b4.z, -b4.w}};
                const float2 w2[2] = {float2{w4.x, w4.y}, float2{w4.z, w4.w}};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float2 a = a2[h];
                    const float2 r = {w2[h].x * a.x - w2[h].y * a.y, w2[h].y * a.x + w2[h].x * a.y};
                    cf[2 * i2 + h] = wrap ? r : a;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < P; ++i) {                  // then R(kr_t): angles add
            const float2 a = cf[i], t = rt[i];
            cf[i] = float2{a.x * t.x - a.y * t.y, a.y * t.x + a.x * t.y};
        }
        __bf16 y1[P], y2[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const float x1 = (i & 1) ? hi_bf16(x1w[i >> 1]) : lo_bf16(x1w[i >> 1]);
            const float x2 = (i & 1) ? hi_bf16(x2w[i >> 1]) : lo_bf16(x2w[i >> 1]);
            y1[i] = (__bf16)(x1 * cf[i].x - x2 * cf[i].y);
            y2[i] = (__bf16)(x2 * cf[i].x + x1 * cf[i].y);
        }
        // dims kr_i .. (16-byte column kr_i / 8) and + D/2 (column + D/16)
        unsigned char* d1 = tile + 16 * k_pos<D>(kr_t, kr_i / 8) + 2 * (kr_i % 8);
        unsigned char* d2 = tile + 16 * k_pos<D>(kr_t, (kr_i + D / 2) / 8) + 2 * (kr_i % 8);
        if constexpr (P == 8) {
            bf16x8 v1, v2;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v1[i] = y1[i];
                v2[i] = y2[i];
            }
            *(bf16x8*)d1 = v1;
            *(bf16x8*)d2 = v2;
        } else {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 v1, v2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v1[i] = y1[i];
                v2[i] = y2[i];
            }
            *(bf16x4*)d1 = v1;
            *(bf16x4*)d2 = v2;
        }
    };

    // Step -1: the rotation of local visit 0 (nothing to compute yet); K(0)
    // (and everything issued before it) has landed once at most K(1) and V(0)
    // are outstanding.
    {
        // everything issued so far: K(0), and the new tokens' stores where
        // they overlapped the first loads (unconditional, so that the
        // compiler knows no store is pending inside the walk)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();                  // every wave's share
        __builtin_amdgcn_sched_barrier(0);
        lds_fence();
        if (n_mine > 2) issue_k(2, ring_k_u + 2 * PB::kKC);
        if (n_mine > 1) issue_v(1, ring_v_u + PB::kV);
        if (n_mine > 0) {
            // the first visit of the ring (rho = -t_o) and prefix visits (rho < 0)
            // compose R(rho) from the conjugate of row |rho|
            const int kv = kvis(0);
            rotate(ring_k, tiles, kv == 0 || (PRE && kv >= c.n_roll), kv == 0 && c.t_o > 0);
        }
        __builtin_amdgcn_s_waitcnt(kLgkm0);
    }

    // queries rotated once, with the softmax scale folded into the rotation
    // (one bf16 rounding, as without it), into MFMA B operands (zero rows pad)
    bf16x8 qb[NW][KK];
    int rq_col[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int row = row0 + 16 * (wave + 4 * w) + n;
        float4 qc[HP][4];
        lds_coef<D>(lds_qc + (row < rows ? row / G : 0) * D * 4, gq, qc);
#pragma unroll
        for (int kk = 0; kk < HP; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float4& f = qc[kk][j];
                f = float4{f.x * c.scale_log2, f.y * c.scale_log2, f.z * c.scale_log2, f.w * c.scale_log2};
            }
        rotate_row<D>(qc, qr[w], qb[w]);
        if (row >= rows) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) qb[w][kk][e] = (__bf16)0.f;
        }
        rq_col[w] = row < rows ? c.rq + row / G : -1;
    }

    // Step s: K(s + 1) and V(s) have landed once at most K(s + 2) and V(s + 1)
    // (issued by step s - 1, where those visits exist) are outstanding; after
    // the barrier every wave is done with step s - 1, so K slot s % 3 (rotated
    // there) and V slot (s - 1) % 3 (used there) take K(s + 3) and V(s + 2).
    // Slot and tile indices repeat every 6 steps; S = s % 6 is a compile-time
    // constant.
    auto step = [&](auto sc, int s) {
        constexpr int S = decltype(sc)::value;
        const bool do_r = s + 1 < n_mine, do_c = s < n_mine;
        if (do_c) {
            const int after = (s + 2 < n_mine ? PB::nK : 0) + (do_r ? PB::nV : 0);
            if (after == PB::nK + PB::nV) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PB::nK + PB::nV));
            else if (after == PB::nV) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PB::nV));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        lds_fence();
        if (s + 3 < n_mine) issue_k(s + 3, ring_k_u + (S % 3) * PB::kKC);
        if (s + 2 < n_mine) issue_v(s + 2, ring_v_u + ((S + 2) % 3) * PB::kV);

        const int kv = kvis(s);
        const VisitSrc vs = visit_src(c, kv);
        const int s0 = vs.s0, rho = vs.rho;
        const bool seam = (kv == 0) && (c.t_o > 0);
        const bool cmp = do_c && act0;                 // a wave without query rows only rotates
        // QK^T of visit s first, so that the rotation's VALU work below runs
        // while the MFMAs execute
        floatx4 a0[NW], a1[NW];
        u32x4 vv[NB];
        if (cmp) {
            const unsigned char* tile = tiles + (S % 2) * PB::kT;
            bf16x8 kA[2][KK];
            const u32x4* kt = (const u32x4*)tile;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                kA[0][kk] = __builtin_bit_cast(bf16x8, kt[k_pos<D>(c.tb0, gq + 4 * kk)]);
                kA[1][kk] = __builtin_bit_cast(bf16x8, kt[k_pos<D>(c.tb1, gq + 4 * kk)]);
            }
            const u32x4* lb = (const u32x4*)(ring_v + (S % 3) * PB::kV) + lane;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) vv[nb] = lb[nb * 64];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                a0[w] = floatx4{0.f, 0.f, 0.f, 0.f};
                a1[w] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (w == 1 && !act1) continue;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    a0[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[0][kk], qb[w][kk], a0[w], 0, 0, 0);
                    a1[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[1][kk], qb[w][kk], a1[w], 0, 0, 0);
                }
            }
        }
        if (do_r)
            rotate(ring_k + ((S + 1) % 3) * PB::kKC, tiles + ((S + 1) % 2) * PB::kT, PRE && kvis(s + 1) >= c.n_roll, false);
        if (cmp) {
            const bool full =
                vs.pre ? (s0 + kTile <= c.F) : ((kv != 0) && (rho + kTile <= c.rq + 1) && (s0 + kTile <= W));
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                if (w == 1 && !act1) break;
                float s8[8] = {a0[w][0], a0[w][1], a0[w][2], a0[w][3], a1[w][0], a1[w][1], a1[w][2], a1[w][3]};
                if (!full) {
                    // branch-free: key index r of each score, then a select
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tt = 8 * gq + e;
                        const int r = rho + tt + ((seam & (tt < c.t_o)) ? W : 0);
                        const bool ok_ring = (r >= 0) & (r <= r_last) & ((rq_col[w] < 0) | (r <= rq_col[w])) &
                                             (s0 + tt < W);
                        const bool ok_pre = s0 + tt < c.F;      // prefix: before every query
                        const bool ok = vs.pre ? ok_pre : ok_ring;
                        s8[e] = ok ? s8[e] : -INFINITY;
                    }
                }
                float mx = s8[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s8[e]);
                mx = max_rows4(mx);
                const bool grow = mx > m[w] + 8.f;       // lazy rescale, wave-uniform branch
                if (__any(grow)) {
                    const float mn = grow ? mx : m[w];
                    const float alpha = fast_exp2(m[w] - mn);
                    l[w] *= alpha;
#pragma unroll
                    for (int i = 0; i < NB; ++i) o[w][i] *= alpha;
                    m[w] = mn;
                }
                bf16x8 pb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pe = fast_exp2(s8[e] - m[w]);
                    l[w] += pe;
                    pb[e] = (__bf16)pe;
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    o[w][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv[nb]), pb,
                                                                       o[w][nb], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(kLgkm0);            // the rotated tile is written
    };
    using std::integral_constant;
    for (int s = 0; s < n_steps; s += 6) {
        step(integral_constant<int, 0>{}, s);
        if (s + 1 < n_steps) step(integral_constant<int, 1>{}, s + 1);
        if (s + 2 < n_steps) step(integral_constant<int, 2>{}, s + 2);
        if (s + 3 < n_steps) step(integral_constant<int, 3>{}, s + 3);
        if (s + 4 < n_steps) step(integral_constant<int, 4>{}, s + 4);
        if (s + 5 < n_steps) step(integral_constant<int, 5>{}, s + 5);
    }
    __builtin_amdgcn_s_waitcnt(0);

    // this block's partial for the wave's rows: O^T element (dim 16 nb + 4 gq + j,
    // column n) in o[w][nb][j]
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        l[w] = sum_rows4(l[w]);
    }
    if constexpr (WG == 2) {
        // group 1 hands its (m, l, O) of every row to group 0 through LDS
        float* xo = (float*)lds_all;                          // [row][D]
        float* xml = xo + 4 * NW * 16 * D;                    // [row][2]
        static_assert((4 * NW * 16 * D + 4 * NW * 16 * 2) * 4 <= WG * PB::kGroup, "merge buffer does not fit");
        __syncthreads();
        if (wg == 1) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int lr = 16 * (wave + 4 * w) + n;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    *(float4*)&xo[lr * D + 16 * nb + 4 * gq] = float4{o[w][nb][0], o[w][nb][1], o[w][nb][2], o[w][nb][3]};
                if (gq == 0) *(float2*)&xml[lr * 2] = float2{m[w], l[w]};
            }
        }
        __syncthreads();
        if (wg == 1) return;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int lr = 16 * (wave + 4 * w) + n;
            const float2 ml1 = *(const float2*)&xml[lr * 2];
            const float mn = fmaxf(m[w], ml1.x);
            const float a0 = exp2f(m[w] - mn), a1 = exp2f(ml1.x - mn);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float4 x = *(const float4*)&xo[lr * D + 16 * nb + 4 * gq];
                o[w][nb][0] = o[w][nb][0] * a0 + x.x * a1;
                o[w][nb][1] = o[w][nb][1] * a0 + x.y * a1;
                o[w][nb][2] = o[w][nb][2] * a0 + x.z * a1;
                o[w][nb][3] = o[w][nb][3] * a0 + x.w * a1;
            }
            l[w] = l[w] * a0 + ml1.y * a1;
            m[w] = mn;
        }
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int row = row0 + 16 * (wave + 4 * w) + n;
        if (row >= rows) continue;
        const int cc = row / G, h = kh * G + (row - cc * G);
        if (n_split == 1) {
            const float inv = 1.f / l[w];
            uint16_t* op = out + (((int64_t)bi * C + cc) * g.hq + h) * D;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j) op[16 * nb + 4 * gq + j] = f32_to_bf16_bits(o[w][nb][j] * inv);
        } else {
            // partials for combine_kernel (launched next on the same stream),
            // stored non-temporal: read once, mostly by blocks on other XCDs
            // (0.3-0.5 us per call less than through the L2)
            const int64_t pr = part_row(g, bi, kh, split, row);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                __builtin_nontemporal_store(floatx4{o[w][nb][0], o[w][nb][1], o[w][nb][2], o[w][nb][3]},
                                            (floatx4*)&g.part_o[pr * D + 16 * nb + 4 * gq]);
            if (gq == 0) __builtin_nontemporal_store(floatx2{m[w], l[w]}, (floatx2*)&g.part_ml[pr * 2]);
        }
    }
}

// Key splits per pair: as many as keep the launch within target_blocks (the
// blocks resident at once; rounding up would leave a second, mostly idle wave
// of blocks), at most one per min_tiles_per_split tiles and kMaxSplits.
int pick_splits(int pairs, int tiles, int target_blocks, int min_tiles_per_split) {
    int sp = target_blocks / pairs;
    int cap = tiles / min_tiles_per_split;
    if (cap < 1) cap = 1;
    if (sp > cap) sp = cap;
    if (sp > kMaxSplits) sp = kMaxSplits;
    if (sp < 1) sp = 1;
    return sp;
}

// Whether any stream of the batch has a pinned prefix (selects the kernel
// instance that walks prefix tiles).
bool any_prefix(const StreamBatch& st) {
    for (int i = 0; i < st.nb; ++i)
        if (st.prefix[i] > 0) return true;
    return false;
}

bool mfma_decode_ok(const Geometry& g) {
    // the walk's buffer offsets are 32-bit: a pair's K (or V) block and the
    // table stay below 2 GiB (windows up to 8M tokens at D = 128)
    return g.elem_bytes == 2 && g.group <= 16 && (g.d == 64 || g.d == 128) &&
           (int64_t)g.pair_slots * g.d * 2 < ((int64_t)1 << 31) &&
           (int64_t)(g.window + g.f_pad + kTablePad) * g.d * 4 < ((int64_t)1 << 31);
}

template <int D, int EB>
hipError_t run_portable(const Geometry& g, int layer, const StreamBatch& st, int n_q, const void* q,
                        void* out, int n_split, hipStream_t s) {
    const int rows = n_q * g.group;
    const int n_rg = (rows + 63) / 64;
    hipLaunchKernelGGL((attn_portable<D, EB>), dim3(n_split * n_rg, g.hkv, st.nb), dim3(256), 0, s, g,
                       layer, st, n_q, q, out, n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_split == 1) return e;
    return launch_combine<D, EB>(g, st.nb, n_q, n_split, out, s);
}

template <int D>
hipError_t run_decode_mfma(const Geometry& g, int layer, const StreamBatch& st, const void* q, void* out,
                           int n_cu, const void* k_new, const void* v_new, hipStream_t s) {
    // one resident block per CU (two waves per SIMD); the split count is
    // rounded down to a power of two: each level of the merge tree adds an
    // exchange round trip (about 0.75 us for one 3B stream, whose four levels
    // take 3.0 of its 10.7 us), so a count between two powers pays the upper
    // one's levels for less walk saved (one 3B stream: 16 splits, one visit
    // per wave, 11.0 us; 8 splits 11.9; 4 splits 15.2)
    int n_split = pick_splits(st.nb * g.hkv, g.w_pad / kTile, n_cu, 4);
    n_split = n_split >= 16 ? 16 : n_split >= 8 ? 8 : n_split >= 4 ? 4 : n_split >= 2 ? 2 : 1;   // the merge tree
                                                                                               // needs a power of two
    // three instances: the method, the method with a pinned prefix in the batch,
    // and the rebase-on-evict variant (which has no prefix)
    // streaming loads when the launch's windows exceed the chip's L2 (8 x 4 MB)
    const bool stream = (int64_t)st.nb * g.hkv * g.w_pad * D * 4 > (int64_t)32 << 20;
    auto kern = g.prerot ? (stream ? decode_mfma<D, true, false, true> : decode_mfma<D, true, false, false>)
              : any_prefix(st) ? (stream ? decode_mfma<D, false, true, true> : decode_mfma<D, false, true, false>)
                               : (stream ? decode_mfma<D, false, false, true> : decode_mfma<D, false, false, false>);
    hipLaunchKernelGGL(kern, dim3(n_split, g.hkv, st.nb), dim3(64 * kDecWaves), 0, s, g, layer, st, (const uint16_t*)q,
                       (uint16_t*)out, n_split, (const uint16_t*)k_new, (const uint16_t*)v_new);
    return hipGetLastError();
}

template <int D, int NW>
hipError_t run_chunk_pipe(const Geometry& g, int layer, const StreamBatch& st, int n_q, const void* q, void* out,
                          int n_cu, hipStream_t s, const void* k_new = nullptr, const void* v_new = nullptr) {
    const int n_rg = (n_q * g.group + 127) / 128;      // row groups of up to 128 query rows
    const int n_split = pick_splits(st.nb * g.hkv * n_rg, g.w_pad / kTile, n_cu, 4);
    // two wave groups per block: two waves per SIMD
    auto kern = any_prefix(st) ? chunk_pipe<D, NW, 2, true> : chunk_pipe<D, NW, 2, false>;
    hipLaunchKernelGGL(kern, dim3(n_split * n_rg, g.hkv, st.nb), dim3(512), 0, s, g, layer, st, n_q,
                       (const uint16_t*)q, (uint16_t*)out, n_split, (const uint16_t*)k_new,
                       (const uint16_t*)v_new);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_split == 1) return e;
    // the splits' partials are merged by a second, chip-wide kernel
    return launch_combine<D, 2>(g, st.nb, n_q, n_split, out, s);
}

// ------------------------------------------------------ window re-prefill ----
// Rebuilds the window of a batch of streams from stored hidden states, the way
// "audio8-asr-infinite-p150" (section "Limitations") rebuilds its rolling
// context by re-prefilling instead of trimming: K = H Wk^T and V = H Wv^T for
// the n tokens of each stream's window (H: [n][hidden], Wk, Wv: [Hkv*D][hidden],
// the layout of a linear layer's weight), bf16 operands on
// v_mfma_f32_16x16x32_bf16 with float32 accumulation, each result rounded once
// to bf16 (nearest even).  Token j of the window goes to ring slot j: K rows as
// appended, V into its transposed 8-slot block.
//
// One block of 16 waves per (256-token tile of one stream, 256 output
// columns); the columns are K's Hkv*D then V's, and a tile may hold both (its
// K columns go to the K ring, its V columns to the V ring).  Waves take 64 x 64
// pieces of the tile (4 x 4 MFMA tiles each).  A (the hidden states) and B (the
// weight rows, both k-contiguous) come into LDS with direct global->LDS buffer
// loads in 64-wide k steps, double-buffered with exact vmcnt waits.  The tile
// size is set by the L2: the walk's operands come from it, not from HBM (each
// token tile is read from HBM once and by every column tile from L2), and a
// 256 x 256 tile moves half the L2 bytes per product of a 256 x 128 one (0.53
// against 0.62 ms per layer, the 256 x 128 form three stages deep).  A staged
// row of 64 k is 8 chunks of 16 bytes, chunk c at position c ^ (row % 8), so
// the operand reads of eight consecutive lanes (rows) fall on distinct banks.
// Rows of the tile past token n re-read token n - 1, so every load stays
// inside the stream's hidden states.  The blocks of one token tile are 8 block
// ids apart, so they run on one XCD and read the token tile from HBM once.
// The epilogue stages the bf16 tile in LDS and writes whole 16-byte chunks: K
// rows, or 8 consecutive slots of one dim for V.  Tokens past n are not
// written, except in V's last 8-slot block, whose slots past n (not live,
// masked out of every attention) get token n - 1's values.
constexpr int kRbM = 256, kRbN = 256, kRbK = 64, kRbStages = 2;
constexpr int kRbStageA = kRbM * kRbK * 2, kRbStageB = kRbN * kRbK * 2;
constexpr int kRbStage = kRbStageA + kRbStageB;
constexpr int kRbOut = kRbN * 2 + 16;                  // LDS bytes per epilogue row
constexpr int kRbLds = kRbStages * kRbStage > kRbM * kRbOut ? kRbStages * kRbStage : kRbM * kRbOut;

__global__ __launch_bounds__(1024, 1) void rebuild_kernel(Geometry g, int layer, StreamBatch st, int n, int hidden,
                                                          const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ wk,
                                                          const uint16_t* __restrict__ wv, int n_row_tiles,
                                                          int n_col_tiles) {
    __shared__ __align__(16) unsigned char lds[kRbLds];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, gq = lane >> 4;
    // block id -> (stream, token tile, column tile): the column tiles of one
    // token tile are 8 ids apart (one XCD)
    const int id = blockIdx.x;
    const int col_t = (id >> 3) % n_col_tiles;
    const int tile = (id & 7) + 8 * ((id >> 3) / n_col_tiles);
    if (tile >= st.nb * n_row_tiles) return;
    const int bi = tile / n_row_tiles, row0 = (tile % n_row_tiles) * kRbM;
    const int D = g.d, kvd = g.hkv * D, col0 = col_t * kRbN;
    // the stream's hidden states, tokens 0 .. n - 1 (n * hidden * 2 < 2^31,
    // checked by the host); the K and V weight rows
    const rsrc_t ra = make_rsrc(h + (int64_t)bi * n * hidden, (uint32_t)n * hidden * 2);
    const rsrc_t rk = make_rsrc(wk, (uint32_t)kvd * hidden * 2);
    const rsrc_t rv = make_rsrc(wv, (uint32_t)kvd * hidden * 2);

    // DMA of one stage: instruction j moves rows 8j .. 8j+7 (1 KiB); lane l
    // writes LDS chunk l % 8 of row 8j + l / 8 with source chunk
    // (l % 8) ^ (l / 8).  32 instructions each for A and B, 2 of each per wave.
    constexpr int nA = kRbM / 8 / 16, nB = kRbN / 8 / 16;
    const uint32_t lane_src = (uint32_t)(16 * ((lane & 7) ^ (lane >> 3)));
    uint32_t va[nA], vb[nB];
    bool bv[nB];                                          // wave-uniform: the rows are V weights
#pragma unroll
    for (int u = 0; u < nA; ++u)
        va[u] = (uint32_t)min(row0 + 8 * (wave * nA + u) + (lane >> 3), n - 1) * hidden * 2 + lane_src;
#pragma unroll
    for (int u = 0; u < nB; ++u) {
        const int c = col0 + 8 * (wave * nB + u);       // 8 rows never straddle K and V (kvd % 128 == 0)
        bv[u] = c >= kvd;
        vb[u] = (uint32_t)(c - (bv[u] ? kvd : 0) + (lane >> 3)) * hidden * 2 + lane_src;
    }
    const uint32_t lds_u = lds_u32(lds);
    auto issue = [&](int kt) {
        const uint32_t st_u = lds_u + (uint32_t)((kt % kRbStages) * kRbStage);
        const uint32_t koff = (uint32_t)kt * kRbK * 2;
#pragma unroll
        for (int u = 0; u < nA; ++u) bdma16<false>(ra, va[u], koff, st_u + 1024 * (wave * nA + u));
#pragma unroll
        for (int u = 0; u < nB; ++u)
            bdma16<false>(bv[u] ? rv : rk, vb[u], koff, st_u + kRbStageA + 1024 * (wave * nB + u));
    };

    // wave (wm, wn) computes rows 64 wm .., columns 64 wn ..
    const int wm = wave >> 2, wn = wave & 3;
    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int swz = n16 & 7;                            // a lane's operand rows are n16 mod 8

    const int n_k = hidden / kRbK;
    issue(0);
    for (int kt = 0; kt < n_k; ++kt) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));       // stage kt, the only one in flight
        __builtin_amdgcn_s_barrier();                   // every wave's share; stage kt - 1 is free
        __builtin_amdgcn_sched_barrier(0);
        lds_fence();
        if (kt + 1 < n_k) issue(kt + 1);
        const int so = (kt % kRbStages) * kRbStage;
#pragma unroll
        for (int kb = 0; kb < kRbK / 32; ++kb) {
            const int ch = 16 * ((4 * kb + gq) ^ swz);
            bf16x8 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = *(const bf16x8*)(lds + so + (64 * wm + 16 * i + n16) * (kRbK * 2) + ch);
                bf[i] = *(const bf16x8*)(lds + so + kRbStageA + (64 * wn + 16 * i + n16) * (kRbK * 2) + ch);
            }
            // C^T tile (i, j): rows = output columns (B), columns = tokens (A),
            // so a lane holds 4 consecutive columns of one token
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(kLgkm0);             // this wave's reads of stage kt are done
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();               // every wave is done with the operand buffers

    // epilogue: bf16 tile [token][column] in LDS, then 16-byte global stores
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // acc[i][j][e]: column 64 wn + 16 j + 4 gq + e, token 64 wm + 16 i + n16
            const int tok = 64 * wm + 16 * i + n16, col = 64 * wn + 16 * j + 4 * gq;
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (__bf16)acc[i][j][e];
            *(bf16x4*)(lds + tok * kRbOut + 2 * col) = v4;
        }
    __syncthreads();
    const int b = st.b0 + bi;
    // K columns: 256 tokens x 32 chunks of 16 bytes
    for (int t = tid; t < kRbM * (kRbN / 8); t += 1024) {
        const int tok = t >> 5, ch = t & 31;
        const int col = col0 + 8 * ch;
        if (col >= kvd || row0 + tok >= n) continue;
        const int kh = col / D, d = col % D;
        uint16_t* dst = (uint16_t*)g.k_ring + ((pair_index(g, layer, b, kh) * g.pair_slots + row0 + tok) * D + d);
        *(u32x4*)dst = *(const u32x4*)(lds + tok * kRbOut + 16 * ch);
    }
    // V columns: 32 groups of 8 slots x 256 columns, 8 consecutive slots of one dim
    for (int t = tid; t < (kRbM / 8) * kRbN; t += 1024) {
        const int grp = t / kRbN, c = t % kRbN;
        const int col = col0 + c;
        if (col < kvd || row0 + 8 * grp >= n) continue;
        const int kh = (col - kvd) / D, d = (col - kvd) % D;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = *(const uint16_t*)(lds + (8 * grp + 2 * e) * kRbOut + 2 * c);
            const uint32_t hi = *(const uint16_t*)(lds + (8 * grp + 2 * e + 1) * kRbOut + 2 * c);
            v[e] = lo | (hi << 16);
        }
        const int slot0 = row0 + 8 * grp;
        uint16_t* dst = (uint16_t*)g.v_ring +
                        ((pair_index(g, layer, b, kh) * (g.pair_slots / 8) + slot0 / 8) * (int64_t)D + d) * 8;
        *(u32x4*)dst = v;
    }
}

// Device record of the rebuilt streams' state: (P, n, n mod W) in `layer`.
__global__ void rebuild_state_kernel(Geometry g, int layer, StreamBatch st, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= st.nb) return;
    DevState s;
    s.next_pos = st.next_pos[i];
    s.length = n;
    s.next_slot = n == g.window ? 0 : n;
    g.state[(int64_t)layer * g.n_streams + st.b0 + i] = s;
}

bool mfma_chunk_ok(const Geometry& g, int n_q) {
    // 32-bit buffer offsets, as for the decode walk
    return g.elem_bytes == 2 && (g.d == 64 || g.d == 128) && n_q >= 2 && n_q <= kMaxPartialQ &&
           (int64_t)g.pair_slots * g.d * 2 < ((int64_t)1 << 31) &&
           (int64_t)(g.window + g.f_pad + kTablePad) * g.d * 4 < ((int64_t)1 << 31);
}

}  // namespace

// ======================================================== static scratch ==
// Split partials of a8r_chunk_attn_static, for callers that cannot allocate:
// one array per GPU, alive until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): the address comes from hipGetSymbolAddress, once per device with
// that device current, and goes into the Geometry the kernels take.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(int device, void** ptr) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != device) e = hipSetDevice(device);
        if (e != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        addr[device] = p;
    }
    *ptr = addr[device];
    return hipSuccess;
}

// ================================================================ launchers ==
hipError_t launch_reset(const Geometry& g, const StreamBatch& after, hipStream_t s) {
    const int threads = g.n_layers * after.nb;
    hipLaunchKernelGGL(reset_kernel, dim3((threads + 255) / 256), dim3(256), 0, s, g, after);
    return hipGetLastError();
}

hipError_t launch_append(const Geometry& g, int layer, const StreamBatch& before, int n_new, const void* k,
                         const void* v, hipStream_t s) {
    if (g.elem_bytes == 2)
        hipLaunchKernelGGL(append_kernel<2>, dim3(before.nb), dim3(256), 0, s, g, layer, before, n_new,
                           (const uint8_t*)k, (const uint8_t*)v);
    else
        hipLaunchKernelGGL(append_kernel<4>, dim3(before.nb), dim3(256), 0, s, g, layer, before, n_new,
                           (const uint8_t*)k, (const uint8_t*)v);
    return hipGetLastError();
}

hipError_t launch_append_prefix(const Geometry& g, int layer, const StreamBatch& st, int n, const void* k,
                                const void* v, hipStream_t s) {
    if (g.elem_bytes == 2)
        hipLaunchKernelGGL(prefix_append_kernel<2>, dim3(st.nb), dim3(256), 0, s, g, layer, st, n,
                           (const uint8_t*)k, (const uint8_t*)v);
    else
        hipLaunchKernelGGL(prefix_append_kernel<4>, dim3(st.nb), dim3(256), 0, s, g, layer, st, n,
                           (const uint8_t*)k, (const uint8_t*)v);
    return hipGetLastError();
}

hipError_t launch_export_prefix(const Geometry& g, int layer, const StreamBatch& st, int n, void* k, void* v,
                                hipStream_t s) {
    if (g.elem_bytes == 2)
        hipLaunchKernelGGL(prefix_export_kernel<2>, dim3(st.nb), dim3(256), 0, s, g, layer, st, n, (uint8_t*)k,
                           (uint8_t*)v);
    else
        hipLaunchKernelGGL(prefix_export_kernel<4>, dim3(st.nb), dim3(256), 0, s, g, layer, st, n, (uint8_t*)k,
                           (uint8_t*)v);
    return hipGetLastError();
}

hipError_t launch_attention(const Geometry& g, int layer, const StreamBatch& now, int n_q, const void* q,
                            void* out, bool allow_mfma, int n_cu, hipStream_t s) {
    if (allow_mfma && n_q == 1 && mfma_decode_ok(g))
        return g.d == 128 ? run_decode_mfma<128>(g, layer, now, q, out, n_cu, nullptr, nullptr, s)
                          : run_decode_mfma<64>(g, layer, now, q, out, n_cu, nullptr, nullptr, s);
    if (allow_mfma && mfma_chunk_ok(g, n_q) && !g.prerot) {
        const bool one = n_q * g.group <= 64;            // one 16-row block per wave suffices
        if (g.d == 128)
            return one ? run_chunk_pipe<128, 1>(g, layer, now, n_q, q, out, n_cu, s)
                       : run_chunk_pipe<128, 2>(g, layer, now, n_q, q, out, n_cu, s);
        return one ? run_chunk_pipe<64, 1>(g, layer, now, n_q, q, out, n_cu, s)
                   : run_chunk_pipe<64, 2>(g, layer, now, n_q, q, out, n_cu, s);
    }
    int sp = 1;
    if (n_q <= kMaxPartialQ) {
        const int n_rg = (n_q * g.group + 63) / 64;
        sp = pick_splits(now.nb * g.hkv * n_rg, (g.w_pad + 15) / 16, 2 * n_cu, 2);
    }
    if (g.elem_bytes == 2)
        return g.d == 128 ? run_portable<128, 2>(g, layer, now, n_q, q, out, sp, s)
                          : run_portable<64, 2>(g, layer, now, n_q, q, out, sp, s);
    return g.d == 128 ? run_portable<128, 4>(g, layer, now, n_q, q, out, sp, s)
                      : run_portable<64, 4>(g, layer, now, n_q, q, out, sp, s);
}

hipError_t launch_rebase(const Geometry& g, int layer, const StreamBatch& before, int n, hipStream_t s) {
    const dim3 grid((g.window + 255) / 256, g.hkv, before.nb);
    if (g.elem_bytes == 2) {
        if (g.d == 128) hipLaunchKernelGGL((rebase_kernel<128, 2>), grid, dim3(256), 0, s, g, layer, before, n);
        else hipLaunchKernelGGL((rebase_kernel<64, 2>), grid, dim3(256), 0, s, g, layer, before, n);
    } else {
        if (g.d == 128) hipLaunchKernelGGL((rebase_kernel<128, 4>), grid, dim3(256), 0, s, g, layer, before, n);
        else hipLaunchKernelGGL((rebase_kernel<64, 4>), grid, dim3(256), 0, s, g, layer, before, n);
    }
    return hipGetLastError();
}

hipError_t launch_append_decode(const Geometry& g, int layer, const StreamBatch& before, const void* k,
                                const void* v, const void* q, void* out, bool allow_mfma, int n_cu,
                                hipStream_t s) {
    if (allow_mfma && mfma_decode_ok(g) && !g.prerot)
        return g.d == 128 ? run_decode_mfma<128>(g, layer, before, q, out, n_cu, k, v, s)
                          : run_decode_mfma<64>(g, layer, before, q, out, n_cu, k, v, s);
    hipError_t e = launch_append(g, layer, before, 1, k, v, s);
    if (e == hipSuccess && g.prerot) e = launch_rebase(g, layer, before, 1, s);
    if (e != hipSuccess) return e;
    StreamBatch now = before;
    for (int i = 0; i < now.nb; ++i) {
        now.next_pos[i] += 1;
        now.length[i] = min(now.length[i] + 1, g.window);
        now.next_slot[i] = now.next_slot[i] + 1 == g.window ? 0 : now.next_slot[i] + 1;
    }
    return launch_attention(g, layer, now, 1, q, out, allow_mfma, n_cu, s);
}

hipError_t launch_rebuild(const Geometry& g, int layer, const StreamBatch& st, int n, int hidden, const void* h,
                          const void* wk, const void* wv, hipStream_t s) {
    const int n_row_tiles = (n + kRbM - 1) / kRbM;
    const int n_col_tiles = 2 * g.hkv * g.d / kRbN;
    const int tiles = st.nb * n_row_tiles;
    const int blocks = 8 * n_col_tiles * ((tiles + 7) / 8);
    hipLaunchKernelGGL(rebuild_kernel, dim3(blocks), dim3(1024), 0, s, g, layer, st, n, hidden, (const uint16_t*)h,
                       (const uint16_t*)wk, (const uint16_t*)wv, n_row_tiles, n_col_tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(rebuild_state_kernel, dim3((st.nb + 127) / 128), dim3(128), 0, s, g, layer, st, n);
    return hipGetLastError();
}

hipError_t launch_append_chunk(const Geometry& g, int layer, const StreamBatch& before, int n, const void* k,
                               const void* v, const void* q, void* out, bool allow_mfma, int n_cu, hipStream_t s) {
    if (n == 1) return launch_append_decode(g, layer, before, k, v, q, out, allow_mfma, n_cu, s);
    // one launch where the chunk kernel runs with a single row group (a second
    // row group would read the new tokens' tiles while the first writes them)
    if (allow_mfma && mfma_chunk_ok(g, n) && !g.prerot && n * g.group <= 128) {
        const bool one = n * g.group <= 64;
        if (g.d == 128)
            return one ? run_chunk_pipe<128, 1>(g, layer, before, n, q, out, n_cu, s, k, v)
                       : run_chunk_pipe<128, 2>(g, layer, before, n, q, out, n_cu, s, k, v);
        return one ? run_chunk_pipe<64, 1>(g, layer, before, n, q, out, n_cu, s, k, v)
                   : run_chunk_pipe<64, 2>(g, layer, before, n, q, out, n_cu, s, k, v);
    }
    hipError_t e = launch_append(g, layer, before, n, k, v, s);
    if (e == hipSuccess && g.prerot) e = launch_rebase(g, layer, before, n, s);
    if (e != hipSuccess) return e;
    StreamBatch now = before;
    for (int i = 0; i < now.nb; ++i) {
        now.next_pos[i] += n;
        now.length[i] = min(now.length[i] + n, g.window);
        now.next_slot[i] = (now.next_slot[i] + n) % g.window;
    }
    return launch_attention(g, layer, now, n, q, out, allow_mfma, n_cu, s);
}

}  // namespace a8r
