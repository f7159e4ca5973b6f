// Decode attention: one new query token per sequence against its KV cache,
// a contiguous cache for full layers and a W-slot ring for sliding layers
// ("Step-3.7-Flash-oQ3e" walkthrough 2.2: a sliding layer's cache keeps only
// W tokens). Keys in the cache are already rotated; the query is rotated here
// at its position L-1. Output is gated per head ("Step-3.7-Flash-oQ3e"
// walkthrough 2.3).
//
// bf16 kernel (gfx950): split-K over the cached positions. A workgroup of 4
// waves owns one (sequence, KV head, split); each wave streams 32-key chunks:
//   S^T (16 keys x 16 heads) = K (16 x D) * Q^T (D x 16)   v_mfma_f32_16x16x32_bf16
//   O^T (D x 16 heads)      += V^T (D x 32 keys) * P^T
// The G query heads of the KV group sit in the 16 MFMA columns, so each K/V
// byte is read from HBM once for all G heads. K is loaded straight into the
// A-operand layout; V is transposed through a per-wave LDS tile. Waves merge
// their (max, sum, output) in LDS; with one split the workgroup writes the
// gated output, otherwise it writes a partial that the merge kernel combines
// by log-sum-exp.
#include <cstdlib>

#include "device_util.h"

namespace hgqa {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kChunk = 32;
constexpr int kDecMinKeysPerBlock = 1024;
constexpr int kDecTargetBlocks = 2048;
constexpr float kLog2eDec = 1.4426950408889634f;

// Waits until at most N vector-memory loads of this wave are outstanding
// (loads retire in order, so everything issued before the last N is done).
template <int N>
__device__ __forceinline__ void vm_wait_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else static_assert(N == 0 || N == 8 || N == 16, "add the count");
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// A V chunk sits in the wave's LDS buffer as [32 keys][D] bf16 rows with the
// 16-byte chunk c of key row k at position c ^ vswz(k): the transposed reads
// (ds_read_b64_tr_b16, 32 lanes = 8 key rows x 2 chunks) hit distinct banks.
template <int D> struct DecSwz;
template <> struct DecSwz<128> {
  static __device__ __forceinline__ int v(int key) { return 2 * (key & 7); }
};
template <> struct DecSwz<64> {
  static __device__ __forceinline__ int v(int key) { return 2 * ((key >> 1) & 3); }
};

template <int D>
struct DecodeLds {
  union {
    uint16_t v[kDecWaves][2][kChunk * D];  // per-wave double-buffered V chunks
    struct {
      float o[kDecWaves][16][D];
      float m[kDecWaves][16];
      float l[kDecWaves][16];
    } mg;
  } u;
  float2 cs[kMaxHalfRotary];
};

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int NS = D / 32;          // k-steps of 32 dims
  constexpr int NDB = D / 16;         // 16-dim blocks of the output
  constexpr int CH = D / 8;           // 16-byte chunks per row
  __shared__ DecodeLds<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int Hkv = a.Hkv, G = a.G;

  const int id = blockIdx.x;
  const int kvh = id % Hkv;
  const int rest = id / Hkv;
  const int split = rest % a.num_splits;
  const int b = rest / a.num_splits;

  int L = a.seq_lens[b];
  L = max(1, min(L, a.max_seq_len));
  const int n_vis = a.sliding ? min(L, a.window) : L;
  const int k_begin = split * a.split_keys;
  if (k_begin >= n_vis) return;
  const int k_end = min(n_vis, k_begin + a.split_keys);

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + (size_t)(b * Hkv + kvh) * a.cap * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + (size_t)(b * Hkv + kvh) * a.cap * D;

  f32x4_t O[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) O[i] = f32x4_t{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sc = a.scale * kLog2eDec;

  // Chunk loads: K straight into the MFMA A-operand layout (lane holds key
  // n16 + 16 kb, dims 32s+8g..+7), V from HBM into the wave's LDS buffer.
  // Keys past the split re-read its last key; their scores are masked.
  constexpr int VDMA = kChunk * CH / 64;  // 1 KB HBM->LDS pieces per V chunk
  auto issue = [&](int key0, u32x4_t (&kf)[2][NS], uint16_t* vbuf) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(key0 + 16 * kb + n16, k_end - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s)
        kf[kb][s] = *reinterpret_cast<const u32x4_t*>(kbase + (size_t)key * D + 32 * s + 8 * g);
    }
#pragma unroll
    for (int i = 0; i < VDMA; ++i) {
      const int P = 64 * i + lane;
      const int row = P / CH, pos = P % CH;
      const int key = min(key0 + row, k_end - 1);
      const uint16_t* src = vbase + (size_t)key * D + 8 * (pos ^ DecSwz<D>::v(row));
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(vbuf + 512 * i), 16, 0, 0);
    }
  };

  // The first chunk starts moving, then q (with each chunk's RoPE partner)
  // and the RoPE frequencies are requested right behind it, so one memory
  // round trip brings all three. (The compiler waits for every outstanding
  // load before a register loaded next to an HBM -> LDS copy is used.)
  constexpr int STEP = kChunk * kDecWaves;
  u32x4_t kfa[2][NS], kfb[2][NS];
  uint16_t* va_buf = sm.u.v[wave][0];
  uint16_t* vb_buf = sm.u.v[wave][1];
  int key0 = k_begin + kChunk * wave;
  if (key0 < k_end) issue(key0, kfa, va_buf);

  const int half = a.rope.half, rdims = a.rope.rdims;
  static_assert(kMaxHalfRotary <= kDecThreads, "one frequency per thread");
  const double freq = tid < half ? a.rope.freq_over_pi[tid] : 0.0;
  const bool hv = n16 < G;
  u32x4_t qraw[NS], qpart[NS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((size_t)b * a.Hq + kvh * G + (hv ? n16 : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d0 = 32 * s + 8 * g;
      const int dp = d0 < half ? d0 + half : (d0 < rdims ? d0 - half : d0);
      qraw[s] = *reinterpret_cast<const u32x4_t*>(qrow + d0);
      qpart[s] = *reinterpret_cast<const u32x4_t*>(qrow + dp);
    }
  }

  // ---- rotate q at position L-1; lane holds head n16, dims 32s+8g..+7
  if (tid < half) sm.cs[tid] = rope_cos_sin(L - 1, freq);
  __syncthreads();
  bf16x8_t qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int d0 = 32 * s + 8 * g;
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(qraw[s][e]);
      x[2 * e + 1] = bf16_hi(qraw[s][e]);
    }
    if (d0 < rdims) {
      const bool first = d0 < half;
      const int i0 = first ? d0 : d0 - half;
      const float sgn = first ? -1.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float2 c0 = sm.cs[i0 + 2 * e], c1 = sm.cs[i0 + 2 * e + 1];
        x[2 * e] = fmaf(x[2 * e], c0.x, sgn * bf16_lo(qpart[s][e]) * c0.y);
        x[2 * e + 1] = fmaf(x[2 * e + 1], c1.x, sgn * bf16_hi(qpart[s][e]) * c1.y);
      }
    }
    u32x4_t packed;
#pragma unroll
    for (int e = 0; e < 4; ++e) packed[e] = hv ? pack_bf16x2(x[2 * e], x[2 * e + 1]) : 0u;
    qf[s] = __builtin_bit_cast(bf16x8_t, packed);
  }

  // V^T operand supplier addresses for ds_read_b64_tr_b16: lane r of each
  // 16-lane group (group g) points at key 4g + r/4 and dims 4(r%4)..+3.
  const int r16 = lane & 15;
  const int vrow0 = 4 * g + (r16 >> 2);
  const int vdim = 4 * (r16 & 3);

  auto compute = [&](int key0, const u32x4_t (&kf)[2][NS], const uint16_t* vbuf) {
    f32x4_t S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      S[kb] = f32x4_t{};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        S[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kb][s]),
                                                         qf[s], S[kb], 0, 0, 0);
    }
    // mask keys past the split; online softmax per head (column n16)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = key0 + 16 * kb + 4 * g + v;
        if (key >= k_end) S[kb][v] = -INFINITY;
        mx = fmaxf(mx, S[kb][v]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * sc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
    u32x4_t pk;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[v] = __builtin_amdgcn_exp2f(fmaf(S[kb][v], sc, -m_new));
        psum += p[v];
      }
      pk[2 * kb] = pack_bf16x2(p[0], p[1]);
      pk[2 * kb + 1] = pack_bf16x2(p[2], p[3]);
    }
    l_run = fmaf(l_run, alpha, psum);
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
    // O^T += V^T P^T: the A operand (16 dims x 32 keys) comes transposed out
    // of LDS, keys 4g..4g+3 then 16+4g..16+4g+3 to match P's order.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 16 * db + vdim;
      const int c = d >> 3, hw = d & 7;
      const int r0 = vrow0, r1 = vrow0 + 16;
      const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(vbuf + r0 * D + 8 * (c ^ DecSwz<D>::v(r0)) + hw));
      const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(vbuf + r1 * D + 8 * (c ^ DecSwz<D>::v(r1)) + hw));
      const i16x8_t va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      O[db] *= alpha;
      O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va), pb, O[db],
                                                       0, 0, 0);
    }
  };

  // Double-buffered chunk loop: the next chunk's loads are in flight while
  // the current one is computed. Unrolled by two so buffers are static.
  while (key0 < k_end) {
    const int k1 = key0 + STEP;
    if (k1 < k_end) {
      issue(k1, kfb, vb_buf);
      vm_wait_keep<2 * NS + VDMA>();
    } else {
      vm_wait_keep<0>();
    }
    compute(key0, kfa, va_buf);
    if (k1 >= k_end) break;
    const int k2 = k1 + STEP;
    __builtin_amdgcn_wave_barrier();  // buffer a is consumed before it is refilled
    if (k2 < k_end) {
      issue(k2, kfa, va_buf);
      vm_wait_keep<2 * NS + VDMA>();
    } else {
      vm_wait_keep<0>();
    }
    compute(k1, kfb, vb_buf);
    __builtin_amdgcn_wave_barrier();
    key0 = k2;
  }

  // ---- merge the waves of this workgroup
  float l_w = l_run + __shfl_xor(l_run, 16, 64);
  l_w += __shfl_xor(l_w, 32, 64);
  __syncthreads();  // every wave is done with its V^T tile (aliased below)
  if (g == 0) {
    sm.u.mg.m[wave][n16] = m_run;
    sm.u.mg.l[wave][n16] = l_w;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 4; ++v) sm.u.mg.o[wave][n16][16 * db + 4 * g + v] = O[db][v];
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += kDecThreads) {
    const int hh = idx / D, d = idx - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sm.u.mg.m[w][hh]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm.u.mg.m[w][hh] - M);
      acc = fmaf(sm.u.mg.o[w][hh][d], f, acc);
      lsum = fmaf(sm.u.mg.l[w][hh], f, lsum);
    }
    const int h = kvh * G + hh;
    if (a.num_splits == 1) {
      const float gv = bf16_to_f32(static_cast<const uint16_t*>(a.gate)[(size_t)b * a.Hq + h]);
      static_cast<uint16_t*>(a.out)[((size_t)b * a.Hq + h) * D + d] =
          f32_to_bf16(sigmoidf_dev(gv) * acc / lsum);
    } else {
      float* part = a.partial + (((size_t)b * a.Hq + h) * a.num_splits + split) * (D + 2);
      part[d] = acc;
      if (d == 0) {
        part[D] = M;
        part[D + 1] = lsum;
      }
    }
  }
}

// Log-sum-exp merge of the splits of one (sequence, head), then the gate.
// grid B*Hq, block D.
template <typename T>
__global__ void decode_merge_kernel(DecodeArgs a) {
  const int id = blockIdx.x;
  const int b = id / a.Hq, h = id - (id / a.Hq) * a.Hq;
  const int D = a.D, d = threadIdx.x;
  int L = a.seq_lens[b];
  L = max(1, min(L, a.max_seq_len));
  const int n_vis = a.sliding ? min(L, a.window) : L;
  const int ns = (n_vis + a.split_keys - 1) / a.split_keys;
  const float* part = a.partial + ((size_t)b * a.Hq + h) * a.num_splits * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part[s * (D + 2) + D]);
  float acc = 0.0f, lsum = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float* p = part + s * (D + 2);
    const float f = __builtin_amdgcn_exp2f(p[D] - M);
    acc = fmaf(p[d], f, acc);
    lsum = fmaf(p[D + 1], f, lsum);
  }
  const size_t gi = (size_t)b * a.Hq + h;
  float gv, res;
  if constexpr (sizeof(T) == 2) {
    gv = bf16_to_f32(static_cast<const uint16_t*>(a.gate)[gi]);
    res = sigmoidf_dev(gv) * acc / lsum;
    static_cast<uint16_t*>(a.out)[gi * D + d] = f32_to_bf16(res);
  } else {
    gv = static_cast<const float*>(a.gate)[gi];
    res = (1.0f / (1.0f + expf(-gv))) * acc / lsum;
    static_cast<float*>(a.out)[gi * D + d] = res;
  }
}

// fp32: one wave per (sequence, query head), plain VALU arithmetic.
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
  __shared__ float qs[128];
  __shared__ float2 cs[kMaxHalfRotary];
  const int lane = threadIdx.x;
  const int id = blockIdx.x;
  const int b = id / a.Hq, h = id - (id / a.Hq) * a.Hq;
  const int D = a.D, kvh = h / a.G;
  int L = a.seq_lens[b];
  L = max(1, min(L, a.max_seq_len));
  const int n_vis = a.sliding ? min(L, a.window) : L;
  const int half = a.rope.half, rdims = a.rope.rdims;
  for (int i = lane; i < half; i += 64) cs[i] = rope_cos_sin(L - 1, a.rope.freq_over_pi[i]);
  __syncthreads();
  const float* q = static_cast<const float*>(a.q) + ((size_t)b * a.Hq + h) * D;
  for (int d = lane; d < D; d += 64) {
    float x = q[d];
    if (d < half) x = fmaf(x, cs[d].x, -q[d + half] * cs[d].y);
    else if (d < rdims) x = fmaf(x, cs[d - half].x, q[d - half] * cs[d - half].y);
    qs[d] = x;
  }
  __syncthreads();
  const float* kc = static_cast<const float*>(a.k_cache) + (size_t)(b * a.Hkv + kvh) * a.cap * D;
  const float* vc = static_cast<const float*>(a.v_cache) + (size_t)(b * a.Hkv + kvh) * a.cap * D;
  float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
  __shared__ float ps[64];
  for (int c0 = 0; c0 < n_vis; c0 += 64) {
    const int slot = c0 + lane;
    float s = -INFINITY;
    if (slot < n_vis) {
      const float* krow = kc + (size_t)slot * D;
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], krow[d], dot);
      s = dot * a.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = expf(m - mn);
    const float p = (slot < n_vis) ? expf(s - mn) : 0.0f;
    l = l * alpha + wave_sum(p);
    ps[lane] = p;
    __syncthreads();
    o0 *= alpha;
    o1 *= alpha;
    const int nk = min(64, n_vis - c0);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = ps[jj];
      const float* vrow = vc + (size_t)(c0 + jj) * D;
      o0 = fmaf(pj, vrow[lane], o0);
      if (lane + 64 < D) o1 = fmaf(pj, vrow[lane + 64], o1);
    }
    m = mn;
    __syncthreads();
  }
  const float gv = static_cast<const float*>(a.gate)[(size_t)b * a.Hq + h];
  const float f = (1.0f / (1.0f + expf(-gv))) / l;
  float* o = static_cast<float*>(a.out) + ((size_t)b * a.Hq + h) * D;
  o[lane] = o0 * f;
  if (lane + 64 < D) o[lane + 64] = o1 * f;
}

DecodePlan plan_decode(Elem e, int B, int Hq, int Hkv, int D, int sliding, int window,
                       int max_seq_len) {
  DecodePlan p{};
  const int n_vis_max = sliding ? (max_seq_len < window ? max_seq_len : window) : max_seq_len;
  if (e == Elem::F32 || n_vis_max <= 0) {
    p.split_keys = n_vis_max > 0 ? n_vis_max : 1;
    p.num_splits = 1;
    p.workspace_bytes = 0;
    return p;
  }
  const long long pairs = (long long)B * Hkv;
  // HGQA_DECODE_SPLIT_KEYS (tuning only) fixes the keys per split.
  if (const char* env = getenv("HGQA_DECODE_SPLIT_KEYS")) {
    long long sk = atoll(env);
    if (sk > 0) {
      sk = (sk + kChunk - 1) / kChunk * kChunk;
      p.split_keys = (int)(sk < n_vis_max ? sk : (n_vis_max + kChunk - 1) / kChunk * kChunk);
      p.num_splits = (n_vis_max + p.split_keys - 1) / p.split_keys;
      p.workspace_bytes = p.num_splits > 1
                              ? (size_t)B * Hq * p.num_splits * (size_t)(D + 2) * sizeof(float)
                              : 0;
      return p;
    }
  }
  // Enough workgroups to fill the chip and balance unequal lengths, but no
  // split below kDecMinKeysPerBlock keys when there are many (sequence, KV
  // head) pairs: short splits cost a merge pass that a 512-slot ring does
  // not repay.
  long long splits = (kDecTargetBlocks + pairs - 1) / pairs;
  const long long min_keys = pairs >= 256 ? kDecMinKeysPerBlock : kDecWaves * kChunk;
  const long long max_splits = (n_vis_max + min_keys - 1) / min_keys;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  long long sk = (n_vis_max + splits - 1) / splits;
  sk = (sk + kChunk - 1) / kChunk * kChunk;
  p.split_keys = (int)sk;
  p.num_splits = (int)((n_vis_max + sk - 1) / sk);
  p.workspace_bytes =
      p.num_splits > 1 ? (size_t)B * Hq * p.num_splits * (size_t)(D + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, Elem e, hipStream_t s) {
  if (e == Elem::F32) {
    hipLaunchKernelGGL(decode_f32_kernel, dim3(a.B * a.Hq), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  const unsigned blocks = (unsigned)((long long)a.B * a.num_splits * a.Hkv);
  if (a.D == 128)
    hipLaunchKernelGGL(decode_bf16_kernel<128>, dim3(blocks), dim3(kDecThreads), 0, s, a);
  else
    hipLaunchKernelGGL(decode_bf16_kernel<64>, dim3(blocks), dim3(kDecThreads), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_splits == 1) return err;
  hipLaunchKernelGGL(decode_merge_kernel<uint16_t>, dim3(a.B * a.Hq), dim3(a.D), 0, s, a);
  return hipGetLastError();
}

}  // namespace hgqa
