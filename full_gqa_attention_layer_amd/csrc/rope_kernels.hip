// RoPE kernels that touch each key once:
//  * the prefill pre-pass: rotates K into a head-major copy [B,Hkv,T,D] and
//    writes the (cos, sin) table [T, r/2] that the attention kernel uses to
//    rotate Q while loading it; row t of sequence b sits at absolute position
//    p0(b) + t (p0(b) > 0 for a chunk that continues a cached sequence, and
//    then each sequence gets its own table);
//  * kv_append: rotates new keys at their absolute positions and scatters
//    keys and values into the layer's cache, slot p (full layer) or p mod W
//    (sliding layer ring).
// RoPE pairs dim i with dim i + r/2 for i < r/2 at frequency theta^(-2i/r);
// dims >= r are copied; a base of 0 is the identity ("Step-3.7-Flash-oQ3e"
// walkthrough 2.3; "Muse-Glimmer-30B-6bit" walkthrough, "the RoPE zero value").
#include "device_util.h"

namespace hgqa {

template <typename T> struct ElemIO;
template <> struct ElemIO<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};
template <> struct ElemIO<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};

// Rotated value of element d of one head row x[0..D) whose (cos, sin) for
// pair i sit in cs[i].
template <typename T>
__device__ __forceinline__ float rope_elem(const T* x, int d, int half, int rdims,
                                           const float2* cs) {
  float xv = ElemIO<T>::load(x + d);
  if (d < half) {
    float2 c = cs[d];
    float y = ElemIO<T>::load(x + d + half);
    return fmaf(xv, c.x, -y * c.y);
  }
  if (d < rdims) {
    float2 c = cs[d - half];
    float y = ElemIO<T>::load(x + d - half);
    return fmaf(xv, c.x, y * c.y);
  }
  return xv;
}

constexpr int kPrepassPositions = 8;

// grid (ceil(T / kPrepassPositions), B), block 256.
template <typename T>
__global__ __launch_bounds__(256) void prefill_rope_prepass(PrefillArgs a) {
  __shared__ float2 cs[kPrepassPositions][kMaxHalfRotary];
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kPrepassPositions;
  const int np = min(kPrepassPositions, a.T - t0);
  const int half = a.rope.half;
  const int p0 = prefill_p0(a, b);
  // one table for every sequence of a plain prefill (sequence 0 writes it),
  // one per sequence for a chunk
  const bool write_cs = a.cs_bstride != 0 || b == 0;
  float2* cs_out = a.cs_table + (size_t)b * a.cs_bstride;
  for (int e = threadIdx.x; e < np * half; e += blockDim.x) {
    int tp = e / half, i = e - tp * half;
    float2 c = rope_cos_sin(p0 + t0 + tp, a.rope.freq_over_pi[i]);
    cs[tp][i] = c;
    if (write_cs) cs_out[(size_t)(t0 + tp) * half + i] = c;
  }
  __syncthreads();
  const T* k = static_cast<const T*>(a.k);
  T* kr = static_cast<T*>(a.k_rot);
  const int D = a.D, Hkv = a.Hkv;
  const int per_pos = Hkv * D;
  for (int e = threadIdx.x; e < np * per_pos; e += blockDim.x) {
    int tp = e / per_pos;
    int r = e - tp * per_pos;
    int h = r / D, d = r - h * D;
    int t = t0 + tp;
    const T* row = k + (((size_t)b * a.T + t) * Hkv + h) * D;
    float y = rope_elem<T>(row, d, half, a.rope.rdims, cs[tp]);
    ElemIO<T>::store(kr + (((size_t)b * Hkv + h) * a.T + t) * D + d, y);
  }
}

// bf16 variant: 16-byte chunks (r is a multiple of 16, so a chunk never
// straddles r/2 or r and its RoPE partner is a whole chunk too). A thread's
// first kPrefetch chunks (and their partners) are requested before the
// cos/sin rows are computed, so the loads' latency hides behind the trig.
constexpr int kPrefetch = 4;
template <int D>
__global__ __launch_bounds__(256) void prefill_rope_prepass_bf16(PrefillArgs a) {
  constexpr int CH = D / 8;
  __shared__ float2 cs[kPrepassPositions][kMaxHalfRotary];
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kPrepassPositions;
  const int np = min(kPrepassPositions, a.T - t0);
  const int half = a.rope.half, rdims = a.rope.rdims;
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  uint16_t* kr = static_cast<uint16_t*>(a.k_rot);
  const int Hkv = a.Hkv;
  const int per_pos = Hkv * CH;
  // a chunk appended before its attention reads K from the cache: only the
  // cos/sin rows are needed (and a block past T only pads the V^T rows)
  const int total = (a.keys_in_cache || np <= 0) ? 0 : np * per_pos;

  // chunk e: position t0 + tp, head h, dims d0..d0+7; its source row and the
  // partner chunk's offset (the chunk itself when it is not rotated)
  auto locate = [&](int e, int& tp, int& h, int& d0, const uint16_t*& row) {
    tp = e / per_pos;
    const int r = e - tp * per_pos;
    h = r / CH;
    d0 = (r - h * CH) * 8;
    row = k + (((size_t)b * a.T + t0 + tp) * Hkv + h) * D;
  };
  auto partner = [&](int d0) { return d0 < half ? d0 + half : (d0 < rdims ? d0 - half : d0); };
  // The frequencies of this thread's (at most two) cos/sin entries come
  // first: loads retire in issue order, and the trig must not wait for K.
  static_assert(kPrepassPositions * kMaxHalfRotary <= 2 * 256, "two cos/sin entries per thread");
  const int ntrig = np * half;
  const int e0 = threadIdx.x, e1 = threadIdx.x + 256;
  const double f0 = e0 < ntrig ? a.rope.freq_over_pi[e0 % max(half, 1)] : 0.0;
  const double f1 = e1 < ntrig ? a.rope.freq_over_pi[e1 % max(half, 1)] : 0.0;
  u32x4_t raw[kPrefetch] = {}, praw[kPrefetch] = {};
#pragma unroll
  for (int c = 0; c < (total > 0 ? kPrefetch : 0); ++c) {
    // clamped, so the loads form one straight run (a thread past the end
    // re-reads the last chunk and stores nothing)
    const int e = min((int)threadIdx.x + 256 * c, total - 1);
    int tp, h, d0;
    const uint16_t* row;
    locate(e, tp, h, d0, row);
    raw[c] = *reinterpret_cast<const u32x4_t*>(row + d0);
    praw[c] = *reinterpret_cast<const u32x4_t*>(row + partner(d0));
  }

  const int p0 = prefill_p0(a, b);
  const bool write_cs = a.cs_bstride != 0 || b == 0;  // see prefill_rope_prepass
  float2* cs_out = a.cs_table + (size_t)b * a.cs_bstride;
  auto trig = [&](int e, double f) {
    const int tp = e / half, i = e - tp * half;
    const float2 c = rope_cos_sin(p0 + t0 + tp, f);
    cs[tp][i] = c;
    if (write_cs) cs_out[(size_t)(t0 + tp) * half + i] = c;
  };
  if (e0 < ntrig) trig(e0, f0);
  if (e1 < ntrig) trig(e1, f1);
  __syncthreads();

  auto rotate_store = [&](int e, u32x4_t x, u32x4_t px) {
    int tp, h, d0;
    const uint16_t* row;
    locate(e, tp, h, d0, row);
    if (d0 < rdims) {
      const bool first = d0 < half;
      const int i0 = first ? d0 : d0 - half;
      const float sgn = first ? -1.0f : 1.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float2 c0 = cs[tp][i0 + 2 * q], c1 = cs[tp][i0 + 2 * q + 1];
        const float y0 = fmaf(bf16_lo(x[q]), c0.x, sgn * bf16_lo(px[q]) * c0.y);
        const float y1 = fmaf(bf16_hi(x[q]), c1.x, sgn * bf16_hi(px[q]) * c1.y);
        x[q] = pack_bf16x2(y0, y1);
      }
    }
    *reinterpret_cast<u32x4_t*>(kr + (((size_t)b * Hkv + h) * a.T + t0 + tp) * D + d0) = x;
  };
#pragma unroll
  for (int c = 0; c < kPrefetch; ++c) {
    const int e = threadIdx.x + 256 * c;
    if (e < total) rotate_store(e, raw[c], praw[c]);
  }
  for (int e = threadIdx.x + 256 * kPrefetch; e < total; e += blockDim.x) {
    int tp, h, d0;
    const uint16_t* row;
    locate(e, tp, h, d0, row);
    rotate_store(e, *reinterpret_cast<const u32x4_t*>(row + d0),
                 *reinterpret_cast<const u32x4_t*>(row + partner(d0)));
  }

  // V^T rows for this block's 8 positions (zeros past T): keys t0 .. t0 + 7
  // are one half of a 16-key group, whose slots hold keys 0-3, 8-11, 4-7,
  // 12-15, so this half's first four keys go to slots 4 hf .. and its last
  // four to slots 8 + 4 hf ..
  if (a.v_t) {
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    const int grp = t0 >> 4, hf = (t0 >> 3) & 1;
    for (int e = threadIdx.x; e < Hkv * D; e += blockDim.x) {
      const int h = e / D, d = e - h * D;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ta = t0 + 2 * i, tb = ta + 1;
        const uint32_t lo = ta < a.T ? v[(((size_t)b * a.T + ta) * Hkv + h) * D + d] : 0u;
        const uint32_t hi = tb < a.T ? v[(((size_t)b * a.T + tb) * Hkv + h) * D + d] : 0u;
        w[i] = lo | (hi << 16);
      }
      uint16_t* row = a.v_t + (((size_t)b * Hkv + h) * D + d) * a.t_pad + 16 * grp;
      *reinterpret_cast<u32x2_t*>(row + 4 * hf) = u32x2_t{w[0], w[1]};
      *reinterpret_cast<u32x2_t*>(row + 8 + 4 * hf) = u32x2_t{w[2], w[3]};
    }
  }
}

hipError_t launch_prefill_prepass(const PrefillArgs& a, Elem e, hipStream_t s) {
  // with V^T the blocks run to t_pad, so its padding keys are written as zeros
  const int tn = a.v_t ? a.t_pad : a.T;
  dim3 grid((tn + kPrepassPositions - 1) / kPrepassPositions, a.B);
  if (e == Elem::F32)
    hipLaunchKernelGGL(prefill_rope_prepass<float>, grid, dim3(256), 0, s, a);
  else if (a.D == 128)
    hipLaunchKernelGGL(prefill_rope_prepass_bf16<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_rope_prepass_bf16<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// grid (tokens, B), block 256. One block per new token that reaches the
// cache: all n_new of them for a full cache, the last min(n_new, W) for a
// ring (earlier ones would be overwritten within this call).
__host__ __device__ inline int append_first_token(const AppendArgs& a) {
  return a.sliding && a.n_new > a.window ? a.n_new - a.window : 0;
}
template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  __shared__ float2 cs[kMaxHalfRotary];
  const int n = blockIdx.x + append_first_token(a), b = blockIdx.y;
  const int start = a.start_pos ? a.start_pos[b] : a.start_uniform;
  const int p = start + n;
  if (p < 0) return;
  int slot;
  if (a.sliding) {
    // Only the last W positions of this call reach the ring: each slot keeps
    // the highest position mapping to it.
    if (p < start + a.n_new - a.window) return;
    slot = p % a.window;
  } else {
    if (p >= a.cap) return;
    slot = p;
  }
  const int half = a.rope.half;
  for (int i = threadIdx.x; i < half; i += blockDim.x)
    cs[i] = rope_cos_sin(p, a.rope.freq_over_pi[i]);
  __syncthreads();
  const int D = a.D, Hkv = a.Hkv;
  const T* kn = static_cast<const T*>(a.k_new) + ((size_t)b * a.n_new + n) * Hkv * D;
  const T* vn = static_cast<const T*>(a.v_new) + ((size_t)b * a.n_new + n) * Hkv * D;
  T* kc = static_cast<T*>(a.k_cache);
  T* vc = static_cast<T*>(a.v_cache);
  for (int e = threadIdx.x; e < Hkv * D; e += blockDim.x) {
    int h = e / D, d = e - h * D;
    size_t dst = (((size_t)b * Hkv + h) * a.cap + slot) * D + d;
    float y = rope_elem<T>(kn + h * D, d, half, a.rope.rdims, cs);
    ElemIO<T>::store(kc + dst, y);
    vc[dst] = vn[e];
  }
}

// bf16 variant: 16-byte chunks, one per thread. The start position, the
// RoPE frequency and the thread's first K chunk (with its partner) and V
// chunk are all requested before anything waits, one round trip for all.
template <int D>
__global__ __launch_bounds__(256) void kv_append_bf16_kernel(AppendArgs a) {
  constexpr int CH = D / 8;
  __shared__ float2 cs[kMaxHalfRotary];
  const int n = blockIdx.x + append_first_token(a), b = blockIdx.y;
  const int tid = threadIdx.x;
  const int half = a.rope.half, rdims = a.rope.rdims;
  const int Hkv = a.Hkv, nch = Hkv * CH;
  typedef __attribute__((address_space(1))) const int global_int;
  int start = a.start_uniform;
  if (a.start_pos) start = *(global_int*)(a.start_pos + b);
  const double f = tid < half ? a.rope.freq_over_pi[tid] : 0.0;
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new) + ((size_t)b * a.n_new + n) * Hkv * D;
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new) + ((size_t)b * a.n_new + n) * Hkv * D;
  auto partner = [&](int d0) { return d0 < half ? d0 + half : (d0 < rdims ? d0 - half : d0); };
  const int e0 = min(tid, nch - 1);  // clamped: one straight run of loads
  const int h0 = e0 / CH, d00 = (e0 - h0 * CH) * 8;
  const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(kn + h0 * D + d00);
  const u32x4_t kp0 = *reinterpret_cast<const u32x4_t*>(kn + h0 * D + partner(d00));
  const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(vn + h0 * D + d00);

  const int p = start + n;
  // No early return: the loads above stay ahead of everything that waits
  // for start_pos; a token that does not reach the cache stores nothing.
  const bool reaches = p >= 0 && (a.sliding ? p >= start + a.n_new - a.window : p < a.cap);
  const int slot = a.sliding ? (p >= 0 ? p % a.window : 0) : p;
  if (tid < half) cs[tid] = rope_cos_sin(p, f);
  __syncthreads();
  if (!reaches) return;
  uint16_t* kc = static_cast<uint16_t*>(a.k_cache);
  uint16_t* vc = static_cast<uint16_t*>(a.v_cache);
  auto put = [&](int h, int d0, u32x4_t x, u32x4_t px, u32x4_t v) {
    if (d0 < rdims) {
      const bool first = d0 < half;
      const int i0 = first ? d0 : d0 - half;
      const float sgn = first ? -1.0f : 1.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float2 c0 = cs[i0 + 2 * q], c1 = cs[i0 + 2 * q + 1];
        const float y0 = fmaf(bf16_lo(x[q]), c0.x, sgn * bf16_lo(px[q]) * c0.y);
        const float y1 = fmaf(bf16_hi(x[q]), c1.x, sgn * bf16_hi(px[q]) * c1.y);
        x[q] = pack_bf16x2(y0, y1);
      }
    }
    const size_t dst = (((size_t)b * Hkv + h) * a.cap + slot) * D + d0;
    *reinterpret_cast<u32x4_t*>(kc + dst) = x;
    *reinterpret_cast<u32x4_t*>(vc + dst) = v;
  };
  if (tid < nch) put(h0, d00, k0, kp0, v0);
  for (int e = tid + 256; e < nch; e += 256) {
    const int h = e / CH, d0 = (e - h * CH) * 8;
    put(h, d0, *reinterpret_cast<const u32x4_t*>(kn + h * D + d0),
        *reinterpret_cast<const u32x4_t*>(kn + h * D + partner(d0)),
        *reinterpret_cast<const u32x4_t*>(vn + h * D + d0));
  }
}

hipError_t launch_kv_append(const AppendArgs& a, Elem e, hipStream_t s) {
  dim3 grid(a.n_new - append_first_token(a), a.B);
  if (e == Elem::BF16 && a.D == 128)
    hipLaunchKernelGGL(kv_append_bf16_kernel<128>, grid, dim3(256), 0, s, a);
  else if (e == Elem::BF16 && a.D == 64)
    hipLaunchKernelGGL(kv_append_bf16_kernel<64>, grid, dim3(256), 0, s, a);
  else if (e == Elem::BF16)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hgqa
