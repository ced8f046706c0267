// Internal definitions shared by the host side (a8r_host.cpp) and the HIP
// kernels (a8r_kernels.hip).  Not part of the public ABI.
//
// Device memory layout of one cache (all regions 256-byte aligned):
//   K ring  [n_layers][n_streams][n_kv_heads][W_pad + F_pad][D]   row per slot:
//            ring slots 0 .. W-1, then the pinned prefix from slot W_pad; a key
//            is stored as appended (the rebase-on-evict variant: rotated to
//            its re-based index)
//   V ring  [n_layers][n_streams][n_kv_heads][(W_pad + F_pad)/8][D][8]   8-slot
//            blocks, transposed inside a block so 8 consecutive slots of one dim
//            are 16 contiguous bytes (the k-operand layout of the PV MFMA)
//   table   [W + F_pad + 32][D/2] float2: (cos, sin)(r * theta^(-2i/D)), built
//            in float64 on the host and rounded once to float32
//   state   [n_layers][n_streams] DevState: a device-side record of every
//            pair's (P, L, S), written by the reset / append kernels and read
//            back only by a8r_get_state to cross-check the host bookkeeping.
//            Kernels take the state they work on from their launch arguments
//            (StreamBatch), filled from the host bookkeeping at call time.
//   scratch split partials: O [rows][D] float32 and (m, l) [rows][2] float32
//            (chunk and portable kernels, merged by combine_kernel), and the
//            decode merge tree's exchange slots, all ones between calls
// W_pad = W rounded up to a multiple of 32 (one MFMA key tile); F_pad = the
// prefix capacity rounded up to 32.  Padding slots are zeroed at creation, never
// written, and never taken as live.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace a8r {

constexpr int kTile = 32;          // keys per MFMA tile (4 aligned 8-slot V blocks)
constexpr int kTablePad = 32;      // extra table rows beyond W
constexpr int kMaxSplits = 16;     // most key splits per (stream, KV head)
constexpr int kMaxPartialQ = 16;   // chunk sizes above this run without splits
constexpr size_t kAlign = 256;
constexpr int kBatch = 128;        // streams per launch (their state travels in the arguments)
constexpr int kMaxGroupMfma = 16;   // query heads per KV head in the MFMA decode kernel
constexpr uint64_t kSlotEmpty = ~(uint64_t)0;   // an exchange slot holding no partial
constexpr int kXSlots = kMaxSplits - 1;         // exchange-slot rows per pair: the nodes of a merge tree
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;   // a8r_chunk_attn_static's split partials, per GPU
constexpr int kMaxDevices = 64;

struct DevState {
    int64_t next_pos;   // absolute position of the next token
    int32_t length;     // live tokens, <= W
    int32_t next_slot;  // slot of the next token
};

// State of up to kBatch consecutive streams [b0, b0 + nb) of one layer, as the
// host bookkeeping holds it when the call is made.
struct StreamBatch {
    int b0, nb;
    int32_t next_slot[kBatch];
    int32_t length[kBatch];
    int32_t prefix[kBatch];   // pinned prefix length F (re-based indices 0 .. F-1; the window follows)
    int64_t next_pos[kBatch];
};

// Everything a kernel needs to find a (layer, stream, kv head) window.
struct Geometry {
    void* k_ring;       // [layer][stream][kv_head][pair_slots][D]: ring slots 0 .. W-1, then the
    void* v_ring;       // pinned prefix at slots w_pad .. w_pad + F - 1 (V: 8-slot blocks transposed)
    const float2* table;
    DevState* state;
    float* part_o;      // split partials: [n_streams][n_kv_heads][kMaxSplits][rows_max][D]
    float* part_ml;     // [n_streams][n_kv_heads][kMaxSplits][rows_max][2]
    uint64_t* part_x;   // decode merge-tree exchange slots, one per output element and tree node:
                        // [kXSlots][n_streams][n_kv_heads][kMaxGroupMfma][D], kSlotEmpty between calls
    int n_layers, n_streams, hq, hkv, group, d, window, w_pad;
    int f_pad;          // prefix capacity rounded up to 32 (0: no prefix)
    int pair_slots;     // w_pad + f_pad: slots per (layer, stream, kv head)
    int elem_bytes;     // 2 (bf16) or 4 (f32)
    int prerot;         // keys are stored rotated to their re-based index (A8R_REBASE_ON_EVICT)
    int rows_max;       // max(1, min(max_chunk, kMaxPartialQ)) * group
    float scale_log2;   // softmax scale * log2(e): scores are kept in base-2 units
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline int64_t pair_index(const Geometry& g, int layer, int b, int kh) {
    return ((int64_t)layer * g.n_streams + b) * g.hkv + kh;
}

// ---- launchers (a8r_kernels.hip); each returns the hipError_t of its launch.
// Device pointers k, v, q, out point at the batch's first stream.
// Writes the device state record of every layer for a batch of reset streams.
hipError_t launch_reset(const Geometry& g, const StreamBatch& after, hipStream_t s);
// A8R_REBASE_ON_EVICT, after launch_append of n tokens (state `before` the
// append): rotates the new tokens' keys to their re-based indices and, where
// the append evicted e tokens, every surviving key by R(-e), in place.
hipError_t launch_rebase(const Geometry& g, int layer, const StreamBatch& before, int n, hipStream_t s);
// Copies n prefix tokens per stream into the pinned prefix of a batch, at
// prefix slots F .. F+n-1 (an import of a8r_export_prefix's output is the same copy).
hipError_t launch_append_prefix(const Geometry& g, int layer, const StreamBatch& st, int n, const void* k,
                                const void* v, hipStream_t s);
// Copies the n prefix tokens of each stream out to k, v [nb][n][Hkv][D].
hipError_t launch_export_prefix(const Geometry& g, int layer, const StreamBatch& st, int n, void* k, void* v,
                                hipStream_t s);
// Copies n_new tokens per stream into the ring; `before` is the state before.
hipError_t launch_append(const Geometry& g, int layer, const StreamBatch& before, int n_new,
                         const void* k, const void* v, hipStream_t s);
// Attention for n_q queries (1 = decode) per stream; `now` is the current state.
hipError_t launch_attention(const Geometry& g, int layer, const StreamBatch& now, int n_q,
                            const void* q, void* out, bool allow_mfma, int n_cu, hipStream_t s);
// One new token per stream appended and attended in one launch where the MFMA
// decode kernel applies (else append + attention); `before` is the state before.
hipError_t launch_append_decode(const Geometry& g, int layer, const StreamBatch& before,
                                const void* k, const void* v, const void* q, void* out,
                                bool allow_mfma, int n_cu, hipStream_t s);
// Window re-prefill: K = H Wk^T, V = H Wv^T for the n tokens of each stream's
// window (H device [nb][n][hidden] bf16, Wk and Wv device [Hkv*D][hidden] bf16),
// written to slots 0 .. n-1 of `layer`; the device state record becomes
// (P, n, n mod W).  Needs bf16, hidden % 64 == 0 and Hkv*D % 128 == 0.
hipError_t launch_rebuild(const Geometry& g, int layer, const StreamBatch& st, int n, int hidden, const void* h,
                          const void* wk, const void* wv, hipStream_t s);
// The device address of the library's static scratch array (kStaticScratchBytes,
// 256-byte aligned) on `device`, looked up once per device and kept.
hipError_t static_scratch(int device, void** ptr);
// n new tokens per stream appended and attended in one launch where the MFMA
// chunk kernel runs with one row group (else append + attention).
hipError_t launch_append_chunk(const Geometry& g, int layer, const StreamBatch& before, int n,
                               const void* k, const void* v, const void* q, void* out,
                               bool allow_mfma, int n_cu, hipStream_t s);

}  // namespace a8r
