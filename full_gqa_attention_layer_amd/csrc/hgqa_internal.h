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
  float2* cs_table;     // workspace: [T, half] (cos, sin)
  int B, T, Hq, Hkv, G, D;
  int sliding, window;
  float scale;          // softmax scale
  RopeArgs rope;
  // Chunked prefill: row t of this call sits at absolute position p0 + t, and
  // keys at positions < p0 come from the layer's cache ([B,Hkv,cap,D], K
  // rotated; slot p, or p mod cap for a ring). Plain prefill: p0 = 0, no cache.
  int p0;
  const void* k_cache;
  const void* v_cache;
  int cap, ring;
};

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
DecodePlan plan_decode(Elem e, int B, int Hq, int Hkv, int D, int sliding,
                       int window, int max_seq_len);
hipError_t launch_decode(const DecodeArgs& a, Elem e, hipStream_t s);

}  // namespace hgqa
