// HIP kernels for rolling-window attention with exact RoPE re-basing (gfx950).
//
// Method ("Audio8 ASR Infinite: What It Actually Takes to Listen Forever",
// flowchart figure and section "Inside the Rolling KV Cache and Exact RoPE
// Re-Basing"): a ring of W slots per (layer, stream, KV head); the live window
// is the last L <= W tokens; its origin is the oldest live token.  A key at
// re-based index r and the query at index r_q are rotated (split-half RoPE,
// "Audio8-ASR-Infinite-mlx", section "Requires a patched mlx-audio-swift";
// theta from "Audio8-ASR-0.1B in audio.cpp", section "Architecture") on read;
// the stored K/V bits are never rewritten.
//
// Kernels:
//   reset_kernel       device copy of the per-pair state after a reset
//   append_kernel      copies new K/V rows into their ring slots and advances
//                      the device state (one block per stream)
//   attn_portable      any dtype / group size / chunk size; LDS-tiled VALU
//   decode_mfma        bf16 decode, QK^T and PV on v_mfma_f32_16x16x32_bf16
//   combine_kernel     merges split-K partials {m, l, O} into the output
//
// Scores are kept in base-2 units (the softmax scale is multiplied by log2 e
// and folded into the query) so every exponential is one v_exp_f32.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "a8r_internal.h"

namespace a8r {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;   // running-max seed: exp2(x - kNegBig) never NaNs

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

__device__ __forceinline__ DevState load_state(const Geometry& g, int layer, int b) {
    return g.state[(int64_t)layer * g.n_streams + b];
}

__device__ __forceinline__ int oldest_slot(const DevState& st, int w) {
    int o = st.next_slot - st.length;
    return o < 0 ? o + w : o;
}

// ---------------------------------------------------------------- reset ----
constexpr int kResetBatch = 128;
struct ResetBatch {
    int b0, nb;
    int64_t pos[kResetBatch];
    int32_t slot[kResetBatch];
};

__global__ void reset_kernel(Geometry g, ResetBatch r) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= g.n_layers * r.nb) return;
    const int layer = t / r.nb, i = t - layer * r.nb;
    DevState s;
    s.next_pos = r.pos[i];
    s.length = 0;
    s.next_slot = r.slot[i];
    g.state[(int64_t)layer * g.n_streams + r.b0 + i] = s;
}

// --------------------------------------------------------------- append ----
// One block per stream: every thread reads the stream's state, the block copies
// n_new x Hkv rows (16 bytes per thread step) into K rows and the transposed V
// blocks, then thread 0 advances the state.  Slot of token j = (S + j) mod W.
template <int EB>
__global__ __launch_bounds__(256) void append_kernel(Geometry g, int layer, int b0, int n_new,
                                                     const uint8_t* __restrict__ k,
                                                     const uint8_t* __restrict__ v) {
    const int bi = blockIdx.x, b = b0 + bi;
    DevState* sp = g.state + (int64_t)layer * g.n_streams + b;
    const DevState st = *sp;
    const int D = g.d, W = g.window;
    constexpr int per16 = 16 / EB;             // elements per 16-byte chunk
    const int chunks = D / per16;
    const int total = n_new * g.hkv * chunks;
    for (int t = threadIdx.x; t < total; t += blockDim.x) {
        const int c = t % chunks;
        const int rest = t / chunks;
        const int kh = rest % g.hkv, j = rest / g.hkv;
        int slot = st.next_slot + j;
        if (slot >= W) slot -= W;
        const int64_t src = ((((int64_t)bi * n_new + j) * g.hkv + kh) * D + (int64_t)c * per16) * EB;
        const int64_t pair = pair_index(g, layer, b, kh);
        // K: row-major row of this slot
        uint8_t* kdst = (uint8_t*)g.k_ring + ((pair * g.w_pad + slot) * D + (int64_t)c * per16) * EB;
        *(u32x4*)kdst = *(const u32x4*)(k + src);
        // V: element d of slot s lives at ((s/8)*D + d)*8 + s%8
        const u32x4 vv = *(const u32x4*)(v + src);
        uint8_t* vblk = (uint8_t*)g.v_ring + ((pair * (g.w_pad / 8) + slot / 8) * (int64_t)D * 8) * EB;
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
    __syncthreads();
    if (threadIdx.x == 0) {
        DevState ns = st;
        ns.next_pos = st.next_pos + n_new;
        ns.length = st.length + n_new > W ? W : st.length + n_new;
        int s = st.next_slot + n_new;
        ns.next_slot = s >= W ? s - W : s;
        *sp = ns;
    }
}

// ------------------------------------------------------ split partials ----
__device__ __forceinline__ int64_t part_row(const Geometry& g, int bi, int kh, int split, int row) {
    return (((int64_t)bi * g.hkv + kh) * kMaxSplits + split) * g.rows_max + row;
}

// One block per output row (stream, query, head); D threads, one per dim.
template <int D, int EB>
__global__ __launch_bounds__(128) void combine_kernel(Geometry g, int n_q, int n_split, void* out) {
    const int o = blockIdx.x;
    const int h = o % g.hq;
    const int c = (o / g.hq) % n_q;
    const int bi = o / (g.hq * n_q);
    const int kh = h / g.group, row = c * g.group + (h - kh * g.group);
    const int d = threadIdx.x;
    float mmax = kNegBig;
    for (int s = 0; s < n_split; ++s) mmax = fmaxf(mmax, g.part_ml[part_row(g, bi, kh, s, row) * 2]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < n_split; ++s) {
        const int64_t pr = part_row(g, bi, kh, s, row);
        const float w = exp2f(g.part_ml[pr * 2] - mmax);
        den += w * g.part_ml[pr * 2 + 1];
        num += w * g.part_o[pr * D + d];
    }
    store_elem<EB>(out, (((int64_t)bi * n_q + c) * g.hq + h) * D + d, num / den);
}

// --------------------------------------------------------- portable path ----
// Block = (split of the key range, KV head, stream) x (group of 64 query rows).
// Rows are (query c, head-in-group hg) = c * G + hg.  Keys are walked in
// re-based order r = 0 .. L-1 (slot = (oldest + r) mod W) in tiles of 16; each
// tile's K rows are rotated by R(r) into LDS; scores, online softmax and PV run
// on VALU with 4 threads per row (4 keys of the tile each for the scores, a
// quarter of the head dims each for PV).
template <int D, int EB>
__global__ __launch_bounds__(256) void attn_portable(Geometry g, int layer, int b0, int n_q,
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
    const int b = b0 + bi, G = g.group, W = g.window;
    const int rows = n_q * G, row0 = rg * RG;
    const DevState st = load_state(g, layer, b);
    const int L = st.length, oldest = oldest_slot(st, W);
    const int64_t pair = pair_index(g, layer, b, kh);
    const void* kring = (const uint8_t*)g.k_ring + pair * g.w_pad * D * EB;
    const void* vring = (const uint8_t*)g.v_ring + pair * g.w_pad * D * EB;

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

    const int n_kt = (L + KT - 1) / KT;
    const int per = (n_kt + n_split - 1) / n_split;
    const int kt0 = split * per, kt1 = min(n_kt, kt0 + per);
    for (int kt = kt0; kt < kt1; ++kt) {
        __syncthreads();
        for (int idx = tid; idx < KT * NP; idx += 256) {
            const int j = idx / NP, i = idx - j * NP, r = kt * KT + j;
            float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
            if (r < L) {
                int slot = oldest + r;
                if (slot >= W) slot -= W;
                const float x1 = load_elem<EB>(kring, (int64_t)slot * D + i);
                const float x2 = load_elem<EB>(kring, (int64_t)slot * D + i + NP);
                const float2 cs = g.table[(int64_t)r * NP + i];
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
            const int j = sub * 4 + jj, r = kt * KT + j;
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
// bf16 decode for one (stream, KV head, split) per block of 4 waves.
//
// The ring is walked in physical 32-slot tiles ("visits"), starting with the
// tile that holds the oldest live slot.  A visit's keys sit at slots s0 + t,
// t in [0, 32); their re-based indices are rho + t for one per-visit rho (the
// first visit may also hold the window's newest keys just before the oldest
// slot: those have index rho + t + W).
//
// Rotation: with R(x) the split-half rotation by index x, the score is
// <R(r_q) q, R(rho + t) k> = <R(r_q - rho) q, R(t) k> because rotations in each
// 2-D plane compose additively and are orthogonal.  So each lane rotates its
// key rows by R(t) (t < 32, from LDS) and the query is rotated once per visit
// by R(r_q - rho) (a table row < W + 32).  All coefficients come from the
// float64-built table; no absolute position enters float arithmetic.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, lane l = 16*gq + n):
//   QK: S^T[key][head] = K_rot[key][dims] * Q_rot^T; A row n of tile half b is
//       key t = 8*(n/4) + 4*b + n%4, so the result gives lane l the scores of
//       keys 8*gq .. 8*gq+7 for head n -- exactly the B operand of PV.
//   PV: O^T[d][head] = V^T[d][keys] * P^T; the A operand is 8 consecutive slots
//       of one dim, i.e. 16 bytes of the transposed 8-slot V block.
// Query heads beyond the group (n >= G) are zero rows and are discarded.
template <int D>
__device__ __forceinline__ void rotate_key_rows(const float2* __restrict__ coef, const u32x4 (&kr)[D / 32],
                                                bf16x8 (&kb)[D / 32]) {
    constexpr int KK = D / 32, HP = KK / 2;
#pragma unroll
    for (int kk = 0; kk < HP; ++kk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float2 cs = coef[32 * kk + e];
            const uint32_t w1 = kr[kk][e >> 1], w2 = kr[kk + HP][e >> 1];
            const float x1 = (e & 1) ? hi_bf16(w1) : lo_bf16(w1);
            const float x2 = (e & 1) ? hi_bf16(w2) : lo_bf16(w2);
            kb[kk][e] = (__bf16)(x1 * cs.x - x2 * cs.y);
            kb[kk + HP][e] = (__bf16)(x2 * cs.x + x1 * cs.y);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void decode_mfma(Geometry g, int layer, int b0,
                                                      const uint16_t* __restrict__ q,
                                                      uint16_t* __restrict__ out, int n_split) {
    constexpr int KK = D / 32, HP = KK / 2, NB = D / 16, NP = D / 2;
    __shared__ float2 rt_lds[kTile * NP];          // R(t), t < 32
    __shared__ float red_o[4][16][D];
    __shared__ float red_ml[4][16][2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int bi = blockIdx.z, kh = blockIdx.y, split = blockIdx.x;
    const int b = b0 + bi, G = g.group, W = g.window;

    for (int idx = tid; idx < kTile * NP; idx += 256) rt_lds[idx] = g.table[idx];

    const DevState st = load_state(g, layer, b);
    const int L = st.length, oldest = oldest_slot(st, W), rq = L - 1;
    const int n_tiles = g.w_pad / kTile;
    const int p0t = oldest / kTile, t_o = oldest - p0t * kTile;
    int n_visit;
    {
        int last = oldest + L - 1;
        if (last < W) {
            n_visit = last / kTile - p0t + 1;
        } else {
            last -= W;
            n_visit = n_tiles - p0t + last / kTile + 1;
            if (n_visit > n_tiles) n_visit = n_tiles;
        }
    }
    const int per = (n_visit + n_split - 1) / n_split;
    const int k0 = split * per, k1 = min(n_visit, k0 + per);

    // the query stays as bf16 bits (the softmax scale is applied to the scores)
    u32x4 qraw[KK];
    if (n < G) {
        const uint16_t* qp = q + ((int64_t)bi * g.hq + kh * G + n) * D + 8 * gq;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qraw[kk] = *(const u32x4*)(qp + 32 * kk);
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qraw[kk] = u32x4{0u, 0u, 0u, 0u};
    }

    const int tb0 = 8 * (n >> 2) + (n & 3), tb1 = tb0 + 4;
    const int64_t pair = pair_index(g, layer, b, kh);
    const uint16_t* kp = (const uint16_t*)g.k_ring + pair * g.w_pad * D;
    const uint16_t* vp = (const uint16_t*)g.v_ring + pair * g.w_pad * D;

    floatx4 o[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = kNegBig, l = 0.f;
    __syncthreads();

    for (int k = k0 + wave; k < k1; k += 4) {
        int p = p0t + k;
        if (p >= n_tiles) p -= n_tiles;
        const int s0 = p * kTile;
        int rho;
        if (k == 0) {
            rho = -t_o;
        } else {
            rho = s0 - oldest;
            if (rho < 0) rho += W;
        }
        u32x4 kr0[KK], kr1[KK], vr[NB];
        {
            const uint16_t* r0 = kp + (int64_t)(s0 + tb0) * D + 8 * gq;
            const uint16_t* r1 = kp + (int64_t)(s0 + tb1) * D + 8 * gq;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                kr0[kk] = *(const u32x4*)(r0 + 32 * kk);
                kr1[kk] = *(const u32x4*)(r1 + 32 * kk);
            }
            const uint16_t* vb = vp + ((int64_t)(p * 4 + gq) * D + n) * 8;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) vr[nb] = *(const u32x4*)(vb + (int64_t)nb * 16 * 8);
        }
        // query rotated by R(r_q - rho)
        bf16x8 qb[KK];
        {
            const float2* ta = g.table + (int64_t)(rq - rho) * NP + 8 * gq;
#pragma unroll
            for (int kk = 0; kk < HP; ++kk) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float2 cs = ta[32 * kk + e];
                    const uint32_t w1 = qraw[kk][e >> 1], w2 = qraw[kk + HP][e >> 1];
                    const float x1 = (e & 1) ? hi_bf16(w1) : lo_bf16(w1);
                    const float x2 = (e & 1) ? hi_bf16(w2) : lo_bf16(w2);
                    qb[kk][e] = (__bf16)(x1 * cs.x - x2 * cs.y);
                    qb[kk + HP][e] = (__bf16)(x2 * cs.x + x1 * cs.y);
                }
            }
        }
        // keys rotated by R(t) (or R(t + W) for the window's newest keys that
        // share the oldest key's tile)
        const bool seam = (k == 0) && (t_o > 0);
        bf16x8 kb0[KK], kb1[KK];
        if (!seam) {
            rotate_key_rows<D>(rt_lds + tb0 * NP + 8 * gq, kr0, kb0);
            rotate_key_rows<D>(rt_lds + tb1 * NP + 8 * gq, kr1, kb1);
        } else {
            const int row0 = tb0 < t_o ? tb0 + W : tb0;
            const int row1 = tb1 < t_o ? tb1 + W : tb1;
            rotate_key_rows<D>(g.table + (int64_t)row0 * NP + 8 * gq, kr0, kb0);
            rotate_key_rows<D>(g.table + (int64_t)row1 * NP + 8 * gq, kr1, kb1);
        }
        floatx4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            sc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb0[kk], qb[kk], sc0, 0, 0, 0);
            sc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb1[kk], qb[kk], sc1, 0, 0, 0);
        }
        const float sl = g.scale_log2;
        float s[8] = {sc0[0] * sl, sc0[1] * sl, sc0[2] * sl, sc0[3] * sl,
                      sc1[0] * sl, sc1[1] * sl, sc1[2] * sl, sc1[3] * sl};
        const bool full = (k != 0) && (rho + kTile <= L) && (s0 + kTile <= W);
        if (!full) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 8 * gq + e;
                int r = rho + t;
                if (seam && t < t_o) r += W;
                const bool ok = (r >= 0) && (r < L) && (s0 + t < W);
                if (!ok) s[e] = -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // lazy rescale: keep the running max unless a score exceeds it by 2^8
        if (mx > m + 8.f) {
            const float alpha = exp2f(m - mx);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < NB; ++i) o[i] *= alpha;
            m = mx;
        }
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = exp2f(s[e] - m);
            l += pe;
            pb[e] = (__bf16)pe;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vr[nb]), pb, o[nb], 0, 0, 0);
    }

    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (n < G) {
        if (gq == 0) {
            red_ml[wave][n][0] = m;
            red_ml[wave][n][1] = l;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) red_o[wave][n][16 * nb + 4 * gq + j] = o[nb][j];
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int h = idx / D, d = idx - h * D;
        float mm = red_ml[0][h][0];
#pragma unroll
        for (int w = 1; w < 4; ++w) mm = fmaxf(mm, red_ml[w][h][0]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = exp2f(red_ml[w][h][0] - mm);
            num += f * red_o[w][h][d];
            den += f * red_ml[w][h][1];
        }
        if (n_split == 1) {
            out[((int64_t)bi * g.hq + kh * G + h) * D + d] = f32_to_bf16_bits(num / den);
        } else {
            const int64_t pr = part_row(g, bi, kh, split, h);
            g.part_o[pr * D + d] = num;
            if (d == 0) {
                g.part_ml[pr * 2] = mm;
                g.part_ml[pr * 2 + 1] = den;
            }
        }
    }
}

int env_splits() {
    static int v = -2;
    if (v == -2) {
        const char* s = getenv("A8R_DEBUG_SPLITS");
        v = s ? atoi(s) : -1;
    }
    return v;
}

}  // namespace

// ================================================================ launchers ==
hipError_t launch_reset(const Geometry& g, int b0, int nb, const int64_t* next_pos,
                        const int32_t* next_slot, hipStream_t s) {
    for (int i0 = 0; i0 < nb; i0 += kResetBatch) {
        ResetBatch r;
        r.b0 = b0 + i0;
        r.nb = min(kResetBatch, nb - i0);
        for (int i = 0; i < r.nb; ++i) {
            r.pos[i] = next_pos[i0 + i];
            r.slot[i] = next_slot[i0 + i];
        }
        const int threads = g.n_layers * r.nb;
        hipLaunchKernelGGL(reset_kernel, dim3((threads + 255) / 256), dim3(256), 0, s, g, r);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_append(const Geometry& g, int layer, int b0, int nb, int n_new, const void* k,
                         const void* v, hipStream_t s) {
    if (g.elem_bytes == 2)
        hipLaunchKernelGGL(append_kernel<2>, dim3(nb), dim3(256), 0, s, g, layer, b0, n_new,
                           (const uint8_t*)k, (const uint8_t*)v);
    else
        hipLaunchKernelGGL(append_kernel<4>, dim3(nb), dim3(256), 0, s, g, layer, b0, n_new,
                           (const uint8_t*)k, (const uint8_t*)v);
    return hipGetLastError();
}

namespace {

template <int D, int EB>
hipError_t run_portable(const Geometry& g, int layer, int b0, int nb, int n_q, const void* q,
                        void* out, int n_split, hipStream_t s) {
    const int rows = n_q * g.group;
    const int n_rg = (rows + 63) / 64;
    hipLaunchKernelGGL((attn_portable<D, EB>), dim3(n_split * n_rg, g.hkv, nb), dim3(256), 0, s, g,
                       layer, b0, n_q, q, out, n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_split == 1) return e;
    hipLaunchKernelGGL((combine_kernel<D, EB>), dim3(nb * n_q * g.hq), dim3(D), 0, s, g, n_q, n_split,
                       out);
    return hipGetLastError();
}

template <int D>
hipError_t run_decode_mfma(const Geometry& g, int layer, int b0, int nb, const void* q, void* out,
                           int n_split, hipStream_t s) {
    hipLaunchKernelGGL((decode_mfma<D>), dim3(n_split, g.hkv, nb), dim3(256), 0, s, g, layer, b0,
                       (const uint16_t*)q, (uint16_t*)out, n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_split == 1) return e;
    hipLaunchKernelGGL((combine_kernel<D, 2>), dim3(nb * g.hq), dim3(D), 0, s, g, 1, n_split, out);
    return hipGetLastError();
}

int pick_splits(int pairs, int tiles, int target_blocks, int min_tiles_per_split) {
    int sp = (target_blocks + pairs - 1) / pairs;
    int cap = tiles / min_tiles_per_split;
    if (cap < 1) cap = 1;
    if (sp > cap) sp = cap;
    if (sp > kMaxSplits) sp = kMaxSplits;
    if (sp < 1) sp = 1;
    return sp;
}

}  // namespace

hipError_t launch_attention(const Geometry& g, int layer, int b0, int nb, int n_q, const void* q,
                            void* out, bool allow_mfma, int n_cu, hipStream_t s) {
    const int pairs = nb * g.hkv;
    const int tiles = g.w_pad / kTile;
    const bool mfma_decode = allow_mfma && n_q == 1 && g.elem_bytes == 2 && g.group <= 16 &&
                             (g.d == 64 || g.d == 128);
    if (mfma_decode) {
        int sp = pick_splits(pairs, tiles, 2 * n_cu, 4);
        if (env_splits() > 0) sp = min(env_splits(), kMaxSplits);
        return g.d == 128 ? run_decode_mfma<128>(g, layer, b0, nb, q, out, sp, s)
                          : run_decode_mfma<64>(g, layer, b0, nb, q, out, sp, s);
    }
    int sp = 1;
    if (n_q <= kMaxPartialQ) {
        const int n_rg = (n_q * g.group + 63) / 64;
        sp = pick_splits(pairs * n_rg, (g.w_pad + 15) / 16, 2 * n_cu, 2);
        if (env_splits() > 0) sp = min(env_splits(), kMaxSplits);
    }
    if (g.elem_bytes == 2)
        return g.d == 128 ? run_portable<128, 2>(g, layer, b0, nb, n_q, q, out, sp, s)
                          : run_portable<64, 2>(g, layer, b0, nb, n_q, q, out, sp, s);
    return g.d == 128 ? run_portable<128, 4>(g, layer, b0, nb, n_q, q, out, sp, s)
                      : run_portable<64, 4>(g, layer, b0, nb, n_q, q, out, sp, s);
}

}  // namespace a8r
