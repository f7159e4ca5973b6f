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
// A-operand layout; V is transposed through a per-wave LDS tile. Each wave
// keeps two chunks in flight (two K register sets, two V tiles). Waves merge
// their (max, sum, output) in LDS; with one split the workgroup writes the
// gated output, otherwise it writes a partial that the merge kernel combines
// by log-sum-exp.
#include "device_util.h"

namespace hgqa {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kChunk = 32;
constexpr int kDecMinKeysPerBlock = 1024;
constexpr int kDecMinKeysFewPairs = 512;
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

// Max and sum over the four 16-lane rows of a wave (the g index of the
// 16x16 MFMA layout) with the row-swap permutes: one swap exchanges rows
// 0<->1 and 2<->3, the other the two 32-lane halves.
__device__ __forceinline__ float rows_max(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t c = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const uint32_t c = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// The V buffer that chunks 0, 2, 4, ... of each wave go through; the wave
// merge at the end reuses it. Chunks 1, 3, 5, ... go through a second LDS
// object, and each wave's cos/sin row sits in a third: the compiler tracks
// HBM -> LDS copies per object, so reading one buffer does not wait for
// copies still in flight into the other.
template <int D>
struct DecodeLds {
  union {
    uint16_t v[kDecWaves][kChunk * D];
    struct {
      float o[kDecWaves][16][D];  // per wave and head, swizzled 16-byte columns
      float m[16][kDecWaves];
      float l[16][kDecWaves];
      float gate[16];  // sigmoid of each head's gate
    } mg;
  } u;
};

// A buffer descriptor over `bytes` from `base`: loads at offsets past it
// return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dec_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int NS = D / 32;          // k-steps of 32 dims
  constexpr int NDB = D / 16;         // 16-dim blocks of the output
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int ROW = 2 * D;          // bytes per cached key
  __shared__ DecodeLds<D> sm;
  __shared__ uint16_t vbuf_odd[kDecWaves][kChunk * D];
  __shared__ float2 cs_rows[kDecWaves][kMaxHalfRotary];

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
  const int nrel = min(n_vis, k_begin + a.split_keys) - k_begin;  // keys of this split

  const size_t head0 = (size_t)(b * Hkv + kvh) * a.cap + k_begin;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + head0 * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + head0 * D;

  f32x4_t O[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) O[i] = f32x4_t{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sc = a.scale * kLog2eDec;

  // Chunk loads through descriptors that end at the split's last key, so a
  // chunk's keys past it read as zeros and every chunk issues the same
  // instructions (no branch around a load: the compiler then waits for
  // exactly the chunk it needs). K goes straight into the MFMA A-operand
  // layout (lane: key n16 + 16 kb, dims 32s + 8g..+7), V from HBM into the
  // wave's LDS buffer in 1 KB pieces.
  constexpr int VDMA = kChunk * CH / 64;
  constexpr int RPP = 64 / CH;                       // key rows per V piece
  const uint32_t koff0 = (uint32_t)(n16 * ROW + 16 * g);
  const uint32_t koff1 = koff0 + 16 * ROW;
  uint32_t voff[2];  // lane offset of V pieces i even / odd (the swizzle differs)
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = RPP * p + lane / CH, pos = lane % CH;
    voff[p] = (uint32_t)((lane / CH) * ROW + 16 * (pos ^ DecSwz<D>::v(row)));
  }
  auto issue = [&](int rel, u32x4_t (&kf)[2][NS], uint16_t* vbuf) {
    // (uniform; readfirstlane keeps the descriptor in scalar registers)
    const int left = __builtin_amdgcn_readfirstlane(min(max(nrel - rel, 0), kChunk) * ROW);
    const __amdgpu_buffer_rsrc_t kr = dec_rsrc(kbase + (size_t)rel * D, left);
    const __amdgpu_buffer_rsrc_t vr = dec_rsrc(vbase + (size_t)rel * D, left);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[0][s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kr, koff0 + 64 * s, 0, 0));
      kf[1][s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kr, koff1 + 64 * s, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < VDMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(vbuf + 512 * i), 16,
                                               voff[i & 1] + (uint32_t)(i * RPP * ROW), 0, 0, 0);
  };

  // The wave's first two chunks start moving, with q (and each q chunk's
  // RoPE partner), the gate and the RoPE frequency between them, so one
  // memory round trip brings the first chunk, q, gate and frequency, and the
  // second chunk is already in flight when the key loop starts.
  constexpr int STEP = kChunk * kDecWaves;
  u32x4_t kfa[2][NS], kfb[2][NS];
  uint16_t* va_buf = sm.u.v[wave];
  uint16_t* vb_buf = vbuf_odd[wave];
  const int rel0 = kChunk * wave;
  issue(rel0, kfa, va_buf);

  const int half = a.rope.half, rdims = a.rope.rdims;
  static_assert(kMaxHalfRotary == 64, "one frequency per lane");
  const double freq = a.rope.freq_over_pi[lane];
  const bool hv = n16 < G;
  const size_t qh = (size_t)b * a.Hq + kvh * G + (hv ? n16 : 0);
  const float gv = bf16_to_f32(static_cast<const uint16_t*>(a.gate)[qh]);
  u32x4_t qraw[NS], qpart[NS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + qh * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d0 = 32 * s + 8 * g;
      const int dp = d0 < half ? d0 + half : (d0 < rdims ? d0 - half : d0);
      qraw[s] = *reinterpret_cast<const u32x4_t*>(qrow + d0);
      qpart[s] = *reinterpret_cast<const u32x4_t*>(qrow + dp);
    }
  }
  issue(rel0 + STEP, kfb, vb_buf);

  // ---- rotate q at position L-1; lane holds head n16, dims 32s+8g..+7.
  // Every wave forms its own cos/sin row (lane i: frequency i), so no
  // workgroup barrier stands between the first loads and the key loop, and
  // the frequency load has no branch around it.
  float2* cs = cs_rows[wave];
  cs[lane] = rope_cos_sin(L - 1, freq);
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
    // Rotated dims take the rotation, the rest pass through; a select, not a
    // branch, so the partner load is not moved into a branch behind the
    // chunks in flight.
    const bool rot = d0 < rdims, first = d0 < half;
    const int i0 = first ? d0 : (rot ? d0 - half : 0);
    const float sgn = first ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 c0 = cs[i0 + 2 * e], c1 = cs[i0 + 2 * e + 1];
      const float y0 = fmaf(x[2 * e], c0.x, sgn * bf16_lo(qpart[s][e]) * c0.y);
      const float y1 = fmaf(x[2 * e + 1], c1.x, sgn * bf16_hi(qpart[s][e]) * c1.y);
      x[2 * e] = rot ? y0 : x[2 * e];
      x[2 * e + 1] = rot ? y1 : x[2 * e + 1];
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

  // One chunk: scores, online softmax, PV. A chunk whose keys all lie past
  // the split (only ever the second of a pair, after a chunk with keys)
  // leaves the state unchanged: its scores are -inf and its V rows zeros.
  auto compute = [&](int rel, const u32x4_t (&kf)[2][NS], const uint16_t* vbuf) {
    f32x4_t S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      S[kb] = f32x4_t{};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        S[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kb][s]),
                                                         qf[s], S[kb], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (rel + 16 * kb + 4 * g + v >= nrel) S[kb][v] = -INFINITY;
        mx = fmaxf(mx, S[kb][v]);
      }
    const float m_new = fmaxf(m_run, rows_max(mx) * sc);
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

  // Chunks in pairs, two in flight: while chunk c is computed, chunk c + 1
  // is arriving; chunk c + 2 is requested into c's buffers once c is done.
  // Every wave issues the same loads each pair, so the waits stay exact. The
  // last pair requests nothing more: requests past the split's keys would
  // only put a round trip between the last chunk and the merge.
  const int nch = rel0 < nrel ? (nrel - rel0 + STEP - 1) / STEP : 0;
  const int npairs = (nch + 1) / 2;
  for (int pr = 0; pr + 1 < npairs; ++pr) {
    const int r = rel0 + 2 * pr * STEP;
    // Scheduling fences around each refill: the buffer's reads (consumed by
    // the products above) are done before its copies are issued, and the
    // next chunk's products stay below, so no wait for that chunk holds the
    // refill up.
    vm_wait_keep<2 * NS + VDMA>();
    compute(r, kfa, va_buf);
    __builtin_amdgcn_sched_barrier(0);
    issue(r + 2 * STEP, kfa, va_buf);
    __builtin_amdgcn_sched_barrier(0);
    vm_wait_keep<2 * NS + VDMA>();
    compute(r + STEP, kfb, vb_buf);
    __builtin_amdgcn_sched_barrier(0);
    issue(r + 3 * STEP, kfb, vb_buf);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (npairs > 0) {
    const int r = rel0 + 2 * (npairs - 1) * STEP;
    vm_wait_keep<2 * NS + VDMA>();
    compute(r, kfa, va_buf);
    vm_wait_keep<0>();
    compute(r + STEP, kfb, vb_buf);
  }

  // ---- merge the waves of this workgroup. A wave's output rows overlay
  // exactly its own buffer a, and the maxima, sums and gates lie past every
  // V buffer, so each wave writes them as soon as its own keys are done.
  static_assert(sizeof(DecodeLds<D>::u.mg.o[0]) == sizeof(DecodeLds<D>::u.v[0]),
                "a wave's output rows overlay its own V buffer");
  static_assert(offsetof(DecodeLds<D>, u.mg.m) >= sizeof(DecodeLds<D>::u.v),
                "the merge's maxima and sums lie past the V buffers");
  const float l_w = rows_sum(l_run);
  __builtin_amdgcn_s_waitcnt(0);  // nothing of this wave is still in flight
  if (g == 0) {
    sm.u.mg.m[n16][wave] = m_run;
    sm.u.mg.l[n16][wave] = l_w;
    if (wave == 0) sm.u.mg.gate[n16] = sigmoidf_dev(gv);
  }
  // Lane (n16, g) holds dims 16db + 4g..+3 of head n16. Each head's row is
  // kept as 16-byte columns XOR-swizzled by the head, so the 16 heads of a
  // write land in distinct banks and a read of consecutive columns of one
  // head stays conflict-free.
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<f32x4_t*>(&sm.u.mg.o[wave][n16][4 * ((4 * db + g) ^ n16)]) = O[db];
  __syncthreads();

  // One thread per (head, 4 dims): weights of the waves from their maxima,
  // the weighted sum of their outputs, then the gate (one split) or a
  // partial for the merge kernel.
  static_assert(kDecWaves == 4, "one float4 of maxima / sums per head");
  constexpr int C4 = D / 4;
  for (int it = tid; it < G * C4; it += kDecThreads) {
    const int hh = it / C4, c4 = it % C4;
    const f32x4_t mw = *reinterpret_cast<const f32x4_t*>(sm.u.mg.m[hh]);
    const f32x4_t lw = *reinterpret_cast<const f32x4_t*>(sm.u.mg.l[hh]);
    const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
    f32x4_t acc = {};
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(mw[w] - M);
      acc += f * *reinterpret_cast<const f32x4_t*>(&sm.u.mg.o[w][hh][4 * (c4 ^ hh)]);
      lsum = fmaf(lw[w], f, lsum);
    }
    const size_t row = (size_t)b * a.Hq + kvh * G + hh;
    if (a.num_splits == 1) {
      const float gs = sm.u.mg.gate[hh];
      u32x2_t packed;
      packed[0] = pack_bf16x2(gs * acc[0] / lsum, gs * acc[1] / lsum);
      packed[1] = pack_bf16x2(gs * acc[2] / lsum, gs * acc[3] / lsum);
      *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + row * D + 4 * c4) = packed;
    } else {
      float* part = a.partial + (row * a.num_splits + split) * (D + 2);
      *reinterpret_cast<float2*>(part + 4 * c4) = make_float2(acc[0], acc[1]);
      *reinterpret_cast<float2*>(part + 4 * c4 + 2) = make_float2(acc[2], acc[3]);
      if (c4 == 0) *reinterpret_cast<float2*>(part + D) = make_float2(M, lsum);
    }
  }
}

// Log-sum-exp merge of the splits of one (sequence, head), then the gate.
// With a few splits (the batched decode's 4): one block of D threads per
// (sequence, head), each thread looping over the splits for its dim.
constexpr int kMergeFewSplits = 4;
__global__ void decode_merge_few_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int D = a.D, d = threadIdx.x;
  int L = a.seq_lens[b];
  L = max(1, min(L, a.max_seq_len));
  const int n_vis = a.sliding ? min(L, a.window) : L;
  const int ns = (n_vis + a.split_keys - 1) / a.split_keys;
  const float* part = a.partial + (size_t)bh * a.num_splits * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part[s * (D + 2) + D]);
  float acc = 0.0f, lsum = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float* p = part + s * (D + 2);
    const float f = __builtin_amdgcn_exp2f(p[D] - M);
    acc = fmaf(p[d], f, acc);
    lsum = fmaf(p[D + 1], f, lsum);
  }
  const float gv = bf16_to_f32(static_cast<const uint16_t*>(a.gate)[bh]);
  static_cast<uint16_t*>(a.out)[(size_t)bh * D + d] = f32_to_bf16(sigmoidf_dev(gv) * acc / lsum);
}

// With more splits (a long context alone has hundreds: a single sequence of
// 64K keys on two KV heads, 129), one thread per dim looping over every split
// is a chain of dependent L2 round trips, so the splits are spread over the
// threads too: one block per (sequence, head, 32 dims) of 16 x NG threads
// (NG = 4, 8 or 16, following the split count), where thread t takes dims
// 2 (t % 16) and 2 (t % 16) + 1 of its 32 and every NG-th split from t / 16;
// the NG split groups then add up through LDS.
constexpr int kMergeDims = 32;
constexpr int kMergeMaxThreads = 256;
__global__ __launch_bounds__(kMergeMaxThreads) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float wave_max[kMergeMaxThreads / 64];
  __shared__ float2 gacc[kMergeMaxThreads];
  __shared__ float gsum[kMergeMaxThreads];
  constexpr int DP = kMergeDims / 2;  // dim pairs per block
  const int D = a.D, nq = D / kMergeDims;
  const int id = blockIdx.x;
  const int bh = id / nq, dq = id - bh * nq;
  const int b = bh / a.Hq;
  const int tid = threadIdx.x, nt = blockDim.x, ng = nt / DP;
  int L = a.seq_lens[b];
  L = max(1, min(L, a.max_seq_len));
  const int n_vis = a.sliding ? min(L, a.window) : L;
  const int ns = (n_vis + a.split_keys - 1) / a.split_keys;
  const int rec = D + 2;  // a split's record: D outputs, its reference, its sum
  const float* part = a.partial + (size_t)bh * a.num_splits * rec;

  // the largest reference over the splits (every split holds a visible key)
  float M = -INFINITY;
  for (int s = tid; s < ns; s += nt) M = fmaxf(M, part[(size_t)s * rec + D]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if ((tid & 63) == 0) wave_max[tid >> 6] = M;
  __syncthreads();
  M = wave_max[0];
  for (int w = 1; w < nt / 64; ++w) M = fmaxf(M, wave_max[w]);

  const int dp = tid % DP, grp = tid / DP;
  const int d = kMergeDims * dq + 2 * dp;
  float2 acc = make_float2(0.0f, 0.0f);
  float lsum = 0.0f;
#pragma unroll 4
  for (int s = grp; s < ns; s += ng) {
    const float* p = part + (size_t)s * rec;
    const float2 ml = *reinterpret_cast<const float2*>(p + D);
    const float2 o = *reinterpret_cast<const float2*>(p + d);
    const float f = __builtin_amdgcn_exp2f(ml.x - M);
    acc.x = fmaf(o.x, f, acc.x);
    acc.y = fmaf(o.y, f, acc.y);
    lsum = fmaf(ml.y, f, lsum);
  }
  gacc[tid] = acc;
  gsum[tid] = lsum;
  __syncthreads();
  if (tid < DP) {
    float2 r = gacc[tid];
    float l = gsum[tid];
    for (int g = 1; g < ng; ++g) {
      const float2 x = gacc[g * DP + tid];
      r.x += x.x;
      r.y += x.y;
      l += gsum[g * DP + tid];
    }
    const float gs = sigmoidf_dev(bf16_to_f32(static_cast<const uint16_t*>(a.gate)[bh])) / l;
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + (size_t)bh * D + d) =
        pack_bf16x2(gs * r.x, gs * r.y);
  }
}

// Threads of a many-split merge block: 16 per split group, 4 to 16 groups.
static int merge_threads(int num_splits) {
  int ng = 4;
  while (ng < 16 && ng < num_splits) ng *= 2;
  return ng * (kMergeDims / 2);
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
                       int max_seq_len, int split_keys_override) {
  DecodePlan p{};
  const int n_vis_max = sliding ? (max_seq_len < window ? max_seq_len : window) : max_seq_len;
  if (e == Elem::F32 || n_vis_max <= 0) {
    p.split_keys = n_vis_max > 0 ? n_vis_max : 1;
    p.num_splits = 1;
    p.workspace_bytes = 0;
    return p;
  }
  const long long pairs = (long long)B * Hkv;
  if (split_keys_override > 0) {
    long long sk = (split_keys_override + kChunk - 1) / kChunk * kChunk;
    p.split_keys = (int)(sk < n_vis_max ? sk : (n_vis_max + kChunk - 1) / kChunk * kChunk);
    p.num_splits = (n_vis_max + p.split_keys - 1) / p.split_keys;
    p.workspace_bytes =
        p.num_splits > 1 ? (size_t)B * Hq * p.num_splits * (size_t)(D + 2) * sizeof(float) : 0;
    return p;
  }
  // Enough workgroups to fill the chip and balance unequal lengths, but no
  // split below kDecMinKeysPerBlock keys when there are many (sequence, KV
  // head) pairs (short splits cost a merge pass that a 512-slot ring does
  // not repay), nor below kDecMinKeysFewPairs otherwise: a split's fixed
  // costs (q rotation, wave merge, partial) outweigh a shorter stream.
  // Measured on one sequence: 65537 keys on 2 KV heads take 30 us in splits
  // of 128 keys, 20 us in splits of 512 or 1024, 29 us in splits of 2048.
  long long splits = (kDecTargetBlocks + pairs - 1) / pairs;
  const long long min_keys = pairs >= 256 ? kDecMinKeysPerBlock : kDecMinKeysFewPairs;
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
  if (a.num_splits <= kMergeFewSplits) {
    hipLaunchKernelGGL(decode_merge_few_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(a.D), 0, s, a);
  } else {
    static_assert(64 % kMergeDims == 0 && 128 % kMergeDims == 0, "whole dim groups");
    hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(a.B * a.Hq * (a.D / kMergeDims))),
                       dim3(merge_threads(a.num_splits)), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hgqa
