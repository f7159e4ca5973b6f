// Internal interface between the C-ABI front end (hgqa_api.cpp) and the HIP
// kernels. Host code only sees these launch functions and argument structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hgqa {

constexpr int kMaxHalfRotary = 64;  // r/2 for head_dim <= 128

// RoPE frequencies of one layer. Pair i (i < half) of a vector at position p
// is rotated by p * theta^(-2i/r); freq_over_pi[i] = theta^(-2i/r) / pi so
// the angle in half-turns is p * freq_over_pi[i], reduced exactly in double.
struct RopeArgs {
  int half;    // r / 2; 0 means no rotation
  int rdims;   // r
  double freq_over_pi[kMaxHalfRotary];
};

// Element types.
enum class Elem { BF16, F32 };

// ---------------------------------------------------------------- prefill
struct PrefillArgs {
  const void* q;        // [B,T,Hq,D]
  const void* k;        // [B,T,Hkv,D], not rotated
  const void* v;        // [B,T,Hkv,D]
  const void* gate;     // [B,T,Hq]
  void* out;            // [B,T,Hq,D]
  void* k_rot;          // workspace: [B,Hkv,T,D] rotated K
  float2* cs_table;     // workspace: [T, half] (cos, sin), or [B, T, half] for chunks
  // A prompt on a full bf16 layer with D = 128: V transposed by the pre-pass,
  // [B, Hkv, D, t_pad] (t_pad = T rounded up to 64, keys past T zero), the
  // keys of each 16-key group in the order the PV product takes them (0-3,
  // 8-11, 4-7, 12-15), so one 16-byte LDS read feeds a product. Null
  // otherwise.
  uint16_t* v_t;
  int t_pad;
  size_t cs_bstride;    // float2 entries between sequences' tables (0: one shared table)
  int B, T, Hq, Hkv, G, D;
  int sliding, window;
  float scale;          // softmax scale
  RopeArgs rope;
  // Chunked prefill: row t of sequence b sits at absolute position
  // p0(b) + t, p0(b) = start_pos[b] clamped to [0, max_end_pos - T], and keys
  // at positions < p0(b) come from the layer's cache ([B,Hkv,cap,D], K
  // rotated; slot p, or p mod cap for a ring). Plain prefill: start_pos NULL
  // (p0 = 0), no cache.
  const int32_t* start_pos;
  int max_end_pos;
  const void* k_cache;
  const void* v_cache;
  int cap, ring;
  // Full-layer chunk whose new keys were appended before the attention: every
  // key, the chunk's too, is read from the cache (slot p), and the pre-pass
  // only writes the cos/sin rows.
  int keys_in_cache;
  int waves;            // bf16 workgroup shape override: 0 automatic, 4 or 8
  // Split over keys (chunks only): each row block's key tiles are cut into
  // num_splits runs of split_tiles; each run writes per-row partials
  // [B, T, Hq, num_splits, D + 4] fp32 (unnormalised output, log2-unit
  // reference, sum) that a merge kernel combines. num_splits 1: no split.
  int num_splits, split_tiles;
  float* partial;
};

// Split plan of a chunk call whose longest sequence ends at max_end_pos
// (split_tiles_override > 0 fixes the tiles per split; tuning only): sets
// a.num_splits and a.split_tiles; returns the partial bytes it needs.
size_t plan_prefill_splits(PrefillArgs& a, Elem e, int max_end_pos, int split_tiles_override);

// Start position of sequence b in a prefill call (device side).
__device__ __forceinline__ int prefill_p0(const PrefillArgs& a, int b) {
  if (!a.start_pos) return 0;
  const int p = a.start_pos[b];
  return p < 0 ? 0 : (p > a.max_end_pos - a.T ? a.max_end_pos - a.T : p);
}

// Rotated-K and cos/sin-table pre-pass, then the attention kernel.
hipError_t launch_prefill(const PrefillArgs& a, Elem e, hipStream_t s);

// ---------------------------------------------------------------- kv append
struct AppendArgs {
  const int32_t* start_pos;  // [B]; NULL: every sequence starts at start_uniform
  int start_uniform;
  const void* k_new;         // [B,n,Hkv,D]
  const void* v_new;         // [B,n,Hkv,D]
  void* k_cache;             // [B,Hkv,cap,D]
  void* v_cache;
  int B, n_new, Hkv, D, cap;
  int sliding, window;
  RopeArgs rope;
};
hipError_t launch_kv_append(const AppendArgs& a, Elem e, hipStream_t s);

// ---------------------------------------------------------------- decode
struct DecodeArgs {
  const void* q;        // [B,Hq,D]
  const void* gate;     // [B,Hq]
  const void* k_cache;  // [B,Hkv,cap,D]
  const void* v_cache;
  const int32_t* seq_lens;  // [B]
  void* out;            // [B,Hq,D]
  float* partial;       // workspace: [B,Hq,num_splits,D+2]
  int B, Hq, Hkv, G, D, cap, max_seq_len;
  int sliding, window;
  int split_keys, num_splits;
  float scale;
  RopeArgs rope;
};

// Split plan for a decode shape (host side; also sizes the workspace).
struct DecodePlan {
  int split_keys;
  int num_splits;
  size_t workspace_bytes;
};
// split_keys_override > 0 fixes the keys per split (tuning only).
DecodePlan plan_decode(Elem e, int B, int Hq, int Hkv, int D, int sliding,
                       int window, int max_seq_len, int split_keys_override);
hipError_t launch_decode(const DecodeArgs& a, Elem e, hipStream_t s);

// The checks, split plan and launch behind attn_decode. With scratch_fn set,
// the per-split partials go to the buffer it returns for the stream's GPU
// (scratch_bytes long) instead of the caller's workspace.
typedef hipError_t (*ScratchFn)(hipStream_t stream, void** ptr);
int decode_call(const void* layer, int batch, const void* q, const void* gate,
                const void* k_cache, const void* v_cache, int cache_capacity,
                const int32_t* seq_lens, int max_seq_len, void* workspace,
                size_t workspace_bytes, void* out, void* stream, ScratchFn scratch_fn,
                size_t scratch_bytes);

}  // namespace hgqa
