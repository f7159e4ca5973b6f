// Prefill attention: causal or sliding-window GQA over a prompt at positions
// 0..T-1, sigmoid-gated per head.
//
// Masks: "Step-3.7-Flash-oQ3e" walkthrough 2.2 (full layers are causal,
// sliding layers also hide keys W or more positions back). GQA: "Step-3.7-
// Flash" model card (64 heads in 8 groups) and "Muse-Glimmer-30B-6bit"
// walkthrough, "GQA 16:1". Gate: "Step-3.7-Flash-oQ3e" walkthrough 2.3 and
// "Muse-Glimmer-30B-6bit" walkthrough, "each layer: double LayerNorm + gated
// attention".
//
// bf16 kernel (gfx950, MFMA): one workgroup of 4 waves owns 128 query rows of
// one KV head, where a row is a (position, query head) pair with the G heads
// of a position adjacent; every K/V tile staged in LDS therefore serves all G
// query heads of its group. Each wave owns 32 rows and computes
//   S^T = K_tile (64 keys x D) * Q^T (D x 32 rows)   v_mfma_f32_32x32x16_bf16
//   O^T += V^T (D x 64 keys) * P^T (64 keys x 32 rows)
// so the softmax probabilities leave the score accumulator already in the
// B-operand layout of the second product. V is stored transposed in LDS with
// its keys permuted to match. K arrives pre-rotated from the pre-pass; Q is
// rotated while it is loaded, from the pre-pass's cos/sin table. Only tiles
// that hold a visible key are visited (sliding layers cost O(T*W)), and only
// tiles that cross the diagonal or the window edge are masked elementwise.
#include "device_util.h"

namespace hgqa {

hipError_t launch_prefill_prepass(const PrefillArgs& a, Elem e, hipStream_t s);

// ------------------------------------------------------------------ bf16
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRows = kWaves * kRowsPerWave;  // 128 query rows per workgroup
constexpr int kBN = 64;                       // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct PrefillLds {
  static constexpr int KSTR = D + 8;    // bf16 per K row (pad: conflict-free b128 reads)
  static constexpr int VSTR = kBN + 8;  // bf16 per V^T row
  uint16_t k[2][kBN * KSTR];
  uint16_t vt[2][D * VSTR];
};

// Column of key k (0..63) of a tile inside a V^T row. Within each group of 16
// keys, the 8 keys one lane half feeds to one 32x32x16 product are adjacent.
__device__ __forceinline__ int vt_col(int k) {
  int kk = k & 15;
  return (k & ~15) + 8 * ((kk >> 2) & 1) + 4 * (kk >> 3) + (kk & 3);
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int KCH = D / 8;                  // 16-byte chunks per row
  constexpr int KLOADS = kBN * KCH / 256;     // K chunks per thread per tile
  constexpr int VITEMS = (kBN / 4) * KCH;     // (key quad, chunk) items per tile
  constexpr int KSTR = PrefillLds<D>::KSTR;
  constexpr int VSTR = PrefillLds<D>::VSTR;
  constexpr int NS = D / 16;                  // k-steps of the score product
  constexpr int NDB = D / 32;                 // 32-wide d blocks of the output
  __shared__ PrefillLds<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int T = a.T, G = a.G, Hq = a.Hq, Hkv = a.Hkv;
  const int TG = T * G;
  const int nrb = (TG + kRows - 1) / kRows;

  // Heaviest row blocks (latest positions) first; the KV head varies fastest
  // so that with 8 KV heads each XCD keeps one head's K/V in its L2.
  const int id = blockIdx.x;
  const int kvh = id % Hkv;
  const int rest = id / Hkv;
  const int b = rest % a.B;
  const int rb = nrb - 1 - rest / a.B;

  const int R0 = rb * kRows;
  const int row = R0 + wave * kRowsPerWave + n;
  const bool row_ok = row < TG;
  const int rowc = row_ok ? row : TG - 1;
  const int t_row = rowc / G;
  const int h = kvh * G + (rowc - t_row * G);

  const int t_lo = R0 / G;
  const int t_hi = (min(R0 + kRows, TG) - 1) / G;
  const int w0 = min(R0 + wave * kRowsPerWave, TG - 1);
  const int w1 = min(R0 + wave * kRowsPerWave + kRowsPerWave - 1, TG - 1);
  const int tw_lo = w0 / G, tw_hi = w1 / G;

  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kr = static_cast<const uint16_t*>(a.k_rot);
  const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v);

  // ---- Q^T fragments, rotated on load: lane holds row n, dims 16s+8g..+7.
  bf16x8_t qf[NS];
  {
    const uint16_t* qrow = qp + ((size_t)(b * T + t_row) * Hq + h) * D;
    const int half = a.rope.half, rdims = a.rope.rdims;
    const float2* csrow = a.cs_table + (size_t)t_row * half;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d0 = 16 * s + 8 * g;
      u32x4_t raw = *reinterpret_cast<const u32x4_t*>(qrow + d0);
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_lo(raw[e]);
        x[2 * e + 1] = bf16_hi(raw[e]);
      }
      if (d0 < rdims) {
        const bool first = d0 < half;
        const int i0 = first ? d0 : d0 - half;
        const float sgn = first ? -1.0f : 1.0f;
        u32x4_t praw = *reinterpret_cast<const u32x4_t*>(qrow + (first ? d0 + half : d0 - half));
        const float4* c4 = reinterpret_cast<const float4*>(csrow + i0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float4 cc = c4[e];  // (cos, sin) of pairs i0+2e, i0+2e+1
          float p0 = bf16_lo(praw[e]), p1 = bf16_hi(praw[e]);
          x[2 * e] = fmaf(x[2 * e], cc.x, sgn * p0 * cc.y);
          x[2 * e + 1] = fmaf(x[2 * e + 1], cc.z, sgn * p1 * cc.w);
        }
      }
      u32x4_t packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) packed[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
      qf[s] = __builtin_bit_cast(bf16x8_t, packed);
    }
  }

  // ---- key range of the workgroup
  const int j_lo = a.sliding ? max(0, t_lo - a.window + 1) : 0;
  const int ntiles = (t_hi + 1 - j_lo + kBN - 1) / kBN;

  const uint16_t* kbase = kr + (size_t)(b * Hkv + kvh) * T * D;
  const uint16_t* vbase = vp + ((size_t)b * T * Hkv + kvh) * D;
  const size_t vstride = (size_t)Hkv * D;

  u32x4_t kreg[KLOADS];
  u32x4_t vreg[4];
  const int vq = tid / KCH, vdc = tid - (tid / KCH) * KCH;

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int c = tid + 256 * u;
      const int key = c / KCH, dc = c - key * KCH;
      const int j = j0 + key;
      kreg[u] = (j < T) ? *reinterpret_cast<const u32x4_t*>(kbase + (size_t)j * D + dc * 8)
                        : u32x4_t{0, 0, 0, 0};
    }
    if (tid < VITEMS) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int j = j0 + 4 * vq + kk;
        vreg[kk] = (j < T) ? *reinterpret_cast<const u32x4_t*>(vbase + (size_t)j * vstride + vdc * 8)
                           : u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int c = tid + 256 * u;
      const int key = c / KCH, dc = c - key * KCH;
      *reinterpret_cast<u32x4_t*>(&sm.k[st][key * KSTR + dc * 8]) = kreg[u];
    }
    if (tid < VITEMS) {
      const int col = vt_col(4 * vq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dims 2e and 2e+1 of the chunk, for the 4 keys of the quad
        const uint32_t k0 = vreg[0][e], k1 = vreg[1][e], k2 = vreg[2][e], k3 = vreg[3][e];
        u32x2_t lo = {(k0 & 0xffffu) | (k1 << 16), (k2 & 0xffffu) | (k3 << 16)};
        u32x2_t hi = {(k0 >> 16) | (k1 & 0xffff0000u), (k2 >> 16) | (k3 & 0xffff0000u)};
        const int d = vdc * 8 + 2 * e;
        *reinterpret_cast<u32x2_t*>(&sm.vt[st][d * VSTR + col]) = lo;
        *reinterpret_cast<u32x2_t*>(&sm.vt[st][(d + 1) * VSTR + col]) = hi;
      }
    }
  };

  f32x16_t O[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) O[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sc = a.scale * kLog2e;

  if (ntiles > 0) {
    load_tile(j_lo);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    const int j0 = j_lo + it * kBN;
    if (it + 1 < ntiles) load_tile(j0 + kBN);

    // S^T for two 32-key blocks
    f32x16_t S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      S[kb] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(
            &sm.k[st][(32 * kb + n) * KSTR + 16 * s + 8 * g]);
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], S[kb], 0, 0, 0);
      }
    }

    // mask only where the tile crosses the diagonal or the window edge
    const bool need_mask = (j0 + kBN - 1 > tw_lo) ||
                           (a.sliding && j0 < tw_hi - a.window + 1);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = j0 + 32 * kb + 8 * (v >> 2) + 4 * g + (v & 3);
          const bool vis = (j <= t_row) && (!a.sliding || t_row - j < a.window);
          if (!vis) S[kb][v] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * sc);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;

    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S[kb][v], sc, -m_use));
        S[kb][v] = p;
        psum += p;
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int i = 0; i < NDB; ++i) O[i] *= alpha;

    // O^T += V^T P^T, 4 k-steps of 16 keys
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1, hh = ks & 1;
      u32x4_t pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(S[kb][8 * hh + 2 * e], S[kb][8 * hh + 2 * e + 1]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(
            &sm.vt[st][(32 * db + n) * VSTR + 16 * ks + 8 * g]);
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, O[db], 0, 0, 0);
      }
    }

    if (it + 1 < ntiles) store_tile(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, gate, store bf16
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (row_ok) {
    const uint16_t* gp = static_cast<const uint16_t*>(a.gate);
    const float gv = bf16_to_f32(gp[(size_t)(b * T + t_row) * Hq + h]);
    const float inv = sigmoidf_dev(gv) / l_tot;
    uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)(b * T + t_row) * Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * g;
        u32x2_t w = {pack_bf16x2(O[db][4 * q4] * inv, O[db][4 * q4 + 1] * inv),
                     pack_bf16x2(O[db][4 * q4 + 2] * inv, O[db][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + d) = w;
      }
  }
}

// ------------------------------------------------------------------ fp32
// One wave per (b, t, h) row, plain VALU arithmetic in fp32 throughout.
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  __shared__ float qs[128];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const size_t id = blockIdx.x;
  const int Hq = a.Hq, T = a.T, D = a.D;
  const int h = (int)(id % Hq);
  const size_t bt = id / Hq;
  const int t = (int)(bt % T);
  const int b = (int)(bt / T);
  const int kvh = h / a.G;
  const int half = a.rope.half, rdims = a.rope.rdims;
  const float* q = static_cast<const float*>(a.q) + id * D;
  const float2* cs = a.cs_table + (size_t)t * half;
  for (int d = lane; d < D; d += 64) {
    float x = q[d];
    if (d < half) x = fmaf(x, cs[d].x, -q[d + half] * cs[d].y);
    else if (d < rdims) x = fmaf(x, cs[d - half].x, q[d - half] * cs[d - half].y);
    qs[d] = x;
  }
  __syncthreads();
  const int lo = a.sliding ? max(0, t - a.window + 1) : 0;
  const float* kr = static_cast<const float*>(a.k_rot) + (size_t)(b * a.Hkv + kvh) * T * D;
  const float* v = static_cast<const float*>(a.v) + ((size_t)b * T * a.Hkv + kvh) * D;
  const size_t vstride = (size_t)a.Hkv * D;
  float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int j0 = lo; j0 <= t; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j <= t) {
      const float* krow = kr + (size_t)j * D;
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], krow[d], dot);
      s = dot * a.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = expf(m - mn);
    const float p = (j <= t) ? expf(s - mn) : 0.0f;
    l = l * alpha + wave_sum(p);
    ps[lane] = p;
    __syncthreads();
    o0 *= alpha;
    o1 *= alpha;
    const int nk = min(64, t - j0 + 1);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = ps[jj];
      const float* vrow = v + (size_t)(j0 + jj) * vstride;
      o0 = fmaf(pj, vrow[lane], o0);
      if (lane + 64 < D) o1 = fmaf(pj, vrow[lane + 64], o1);
    }
    m = mn;
    __syncthreads();
  }
  const float gv = static_cast<const float*>(a.gate)[id];
  const float f = (1.0f / (1.0f + expf(-gv))) / l;
  float* o = static_cast<float*>(a.out) + id * D;
  if (lane < D) o[lane] = o0 * f;
  if (lane + 64 < D) o[lane + 64] = o1 * f;
}

hipError_t launch_prefill(const PrefillArgs& a, Elem e, hipStream_t s) {
  hipError_t err = launch_prefill_prepass(a, e, s);
  if (err != hipSuccess) return err;
  if (e == Elem::F32) {
    const size_t rows = (size_t)a.B * a.T * a.Hq;
    hipLaunchKernelGGL(prefill_f32_kernel, dim3((unsigned)rows), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  const long long TG = (long long)a.T * a.G;
  const long long nrb = (TG + kRows - 1) / kRows;
  const long long blocks = nrb * a.B * a.Hkv;
  if (a.D == 128)
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hgqa
