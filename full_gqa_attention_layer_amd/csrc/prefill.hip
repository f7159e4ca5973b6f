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
// bf16 kernel (gfx950, MFMA): one workgroup of 4 or 8 waves owns 128 or 256
// query rows of one KV head, where a row is a (position, query head) pair with
// the G heads of a position adjacent; every K/V tile staged in LDS therefore
// serves all G query heads of its group. Each wave owns 32 rows and computes
//   S^T = K_tile (64 keys x D) * Q^T (D x 32 rows)   v_mfma_f32_32x32x16_bf16
//   O^T += V^T (D x 64 keys) * P^T (64 keys x 32 rows)
// so the softmax probabilities leave the score accumulator already in the
// B-operand layout of the second product. V sits in LDS as rows and is read
// transposed (ds_read_b64_tr_b16) in P's key order. Tiles move HBM -> LDS
// through two stages, the next tile's copy interleaved with this tile's score
// products, one barrier per tile. K arrives pre-rotated from the pre-pass; Q is
// rotated while it is loaded, from the pre-pass's cos/sin table, and carries
// the softmax scale in log2 units; the score accumulators start from minus
// the row's softmax reference, so exp2 applies to them directly. Only tiles
// that hold a visible key are visited (sliding layers cost O(T*W)), and only
// tiles that cross the diagonal or the window edge are masked elementwise.
#include "device_util.h"

#include <algorithm>
#include <type_traits>

namespace hgqa {

hipError_t launch_prefill_prepass(const PrefillArgs& a, Elem e, hipStream_t s);

// ------------------------------------------------------------------ bf16
constexpr int kRowsPerWave = 32;
constexpr int kBN = 64;                       // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// K and V tiles sit in LDS as [64 keys][D] bf16 rows, unpadded. The 16-byte
// chunk c of key row k is stored at chunk position c ^ swz(k); the global
// loads pick their source chunk so that each lane's 16 bytes land at its own
// position (global_load_lds writes lane l at base + 16 l). The swizzles make
// both readers conflict-free:
//  * K: ds_read_b128, 16 lanes read one chunk of 16 consecutive keys;
//  * V: ds_read_b64_tr_b16, 32 lanes read 4 consecutive keys x 4 chunks.
template <int D> struct Swz;
template <> struct Swz<128> {  // 64-dword rows: only the chunk position moves banks
  static __device__ __forceinline__ int k(int key) { return key & 15; }
  static __device__ __forceinline__ int v(int key) { return 4 * (key & 3); }
};
template <> struct Swz<64> {   // 32-dword rows: odd rows sit 32 banks over
  static __device__ __forceinline__ int k(int key) { return (key >> 1) & 7; }
  static __device__ __forceinline__ int v(int key) { return 4 * ((key >> 1) & 1); }
};
// A V^T tile sits as [128 dims][64 slots] bf16 rows (128 bytes: odd rows 32
// banks over); chunk c of row dim is stored at position c ^ ((dim >> 1) & 7),
// so 16 lanes reading one chunk of 16 consecutive dims hit distinct banks.
struct SwzT {
  static __device__ __forceinline__ int c(int dim) { return (dim >> 1) & 7; }
};

__device__ __forceinline__ void unpack8(u32x4_t raw, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(raw[e]);
    x[2 * e + 1] = bf16_hi(raw[e]);
  }
}
__device__ __forceinline__ bf16x8_t pack8(const float (&x)[8]) {
  u32x4_t packed;
#pragma unroll
  for (int e = 0; e < 4; ++e) packed[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  return __builtin_bit_cast(bf16x8_t, packed);
}
// x_e <- x_e cos_e + sgn * partner_e sin_e for the 8 pairs whose (cos, sin)
// start at cs.
__device__ __forceinline__ void rotate8(float (&x)[8], u32x4_t praw, const float2* cs, float sgn) {
  const float4* c4 = reinterpret_cast<const float4*>(cs);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float4 cc = c4[e];  // (cos, sin) of two consecutive pairs
    x[2 * e] = fmaf(x[2 * e], cc.x, sgn * bf16_lo(praw[e]) * cc.y);
    x[2 * e + 1] = fmaf(x[2 * e + 1], cc.z, sgn * bf16_hi(praw[e]) * cc.w);
  }
}

// Rotates a lane's Q chunks (chunk s = dims 16s+8g..+7) when r/2 = 16 H16:
// chunk s < H16 pairs with chunk s + H16 of the same lane; chunks up to
// 2 H16 rotate, the rest pass through. Every value is then multiplied by
// qscale before its one rounding to bf16.
template <int NS, int H16>
__device__ __forceinline__ void rope_q_inlane(const u32x4_t (&raw)[NS], bf16x8_t (&qf)[NS], int g,
                                              const float2* cs, float qscale) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float x[8];
    unpack8(raw[s], x);
    if constexpr (H16 > 0) {
      if (s < 2 * H16) {
        const bool first = s < H16;
        const int sp = first ? s + H16 : s - H16;
        const int i0 = 16 * (first ? s : s - H16) + 8 * g;
        rotate8(x, raw[sp < NS ? sp : 0], cs + i0, first ? -1.0f : 1.0f);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= qscale;
    qf[s] = pack8(x);
  }
}

// Buffer descriptors give a tile's copies a uniform base, so the fixed 32-bit
// lane offsets need no per-tile vector arithmetic. bytes bounds the copy.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, lds_void_t* dst, uint32_t voff,
                                              uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

constexpr int kCsFloat2 = 1024;  // cos/sin rows of one row block: 8 KB

// One stage holds a K tile and a V tile; the kernel keeps its two stages as
// two LDS objects (see the tile loop). With 4 waves (128 rows), stage 1
// first holds the block's Q rows (128 x D bf16 = kBN x 2D) and stage 0
// finally the output rows; with 8 waves (256 rows, one workgroup per CU) a
// separate area holds first Q, then the output.
template <int D>
struct PrefillStage {
  uint16_t k[kBN * D];
  uint16_t v[kBN * D];
};
template <int D, int KW>
struct PrefillLds {
  uint16_t qo[KW > 4 ? KW * kRowsPerWave * D : 8];
  float2 cs[KW > 4 ? 2 * kCsFloat2 : kCsFloat2];
};

// kCache: 0 for a prompt; 1 for a chunk, keys before position p0 from the
// cache and the chunk's own keys from k and v; 2 for a chunk of a full layer
// that was appended first, every key from the cache.
// KW: waves per workgroup (4: two workgroups per CU; 8: one, every K/V tile
// serving twice the rows). SL: sliding-window mask (else causal only).
template <int D, int kCache, int KW, bool SL>
__global__ __launch_bounds__(KW * 64, 8 / KW) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int kWaves = KW;
  constexpr int kRows = kWaves * kRowsPerWave;  // query rows per workgroup
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int PER_WAVE = CH / kWaves;       // 1 KB loads per wave per operand per tile
  static_assert(CH % kWaves == 0, "each wave moves whole 1 KB pieces");
  static_assert(2 * PER_WAVE < 16, "tile-0 pieces fit the 4-bit vmcnt field");
  constexpr int NS = D / 16;                  // k-steps of the score product
  constexpr int NDB = D / 32;                 // 32-wide d blocks of the output
  __shared__ PrefillLds<D, KW> sm;
  __shared__ PrefillStage<D> stage0, stage1;
  auto stg = [&](int i) -> PrefillStage<D>& { return i ? stage1 : stage0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
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
  const int rest2 = rest / a.B;
  const int split = kCache ? rest2 % a.num_splits : 0;  // key split (chunks only)
  const int rb = nrb - 1 - (kCache ? rest2 / a.num_splits : rest2);

  // Rows of the block split into (position, head in group). R0 = t0 G + hg0
  // once; a local row r then needs only the small quotient (hg0 + r) / G,
  // taken in fp32 as floor((y + 1/2) / G): exact for y < 2^21, because the
  // half keeps y / G + 1/(2G) at least 1/(2G) away from an integer, far
  // more than the product's rounding error. Integer division by a runtime G
  // would cost some 30 VALU instructions per use.
  const int R0 = rb * kRows;
  const int t0 = R0 / G, hg0 = R0 - t0 * G;
  const int nrows = min(kRows, TG - R0);  // rows of this block, >= 1
  const float inv_g = 1.0f / (float)G, half_inv_g = 0.5f * inv_g;
  auto split_local = [&](int r, int& dt, int& hg) {
    const int y = hg0 + r;
    dt = (int)fmaf((float)y, inv_g, half_inv_g);
    hg = y - (int)__umul24(dt, G);
  };
  auto pos_of_local = [&](int r) {  // position offset from t0 of local row r, uniform r
    int dt, hg;
    split_local(r, dt, hg);
    return __builtin_amdgcn_readfirstlane(dt);
  };

  const int rl = wave * kRowsPerWave + n;
  const bool row_ok = rl < nrows;
  const bool wave_rows = wave * kRowsPerWave < nrows;  // uniform per wave
  int dt_row, hg_row;
  split_local(min(rl, nrows - 1), dt_row, hg_row);
  const int t_row = t0 + dt_row;

  const int t_lo = t0;
  const int t_hi = t0 + pos_of_local(nrows - 1);
  // Masks and key ranges use absolute positions: row t of this call sits at
  // p0 + t, and so does key t of this call.
  const int p0 = kCache ? prefill_p0(a, b) : 0;
  const int tw_lo = p0 + t0 + pos_of_local(min(wave * kRowsPerWave, nrows - 1));
  const int tw_hi = p0 + t0 + pos_of_local(min(wave * kRowsPerWave + kRowsPerWave - 1, nrows - 1));
  const int t_abs = p0 + t_row;

  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kr = static_cast<const uint16_t*>(a.k_rot);
  const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v);
  // Memory row of (position t0, first head of the group); a row of the block
  // sits dt Hq + hg rows further on.
  const size_t blk_row = (size_t)(b * T + t0) * Hq + kvh * G;

  // ---- key range of the workgroup (absolute positions)
  int j_lo = SL ? max(0, p0 + t_lo - a.window + 1) : 0;
  int ntiles = (p0 + t_hi + 1 - j_lo + kBN - 1) / kBN;
  const int j_last = p0 + T - 1;

  // A split takes tiles [split * split_tiles, ...) of the block's range and
  // writes partials; a split past the range marks its rows empty.
  const size_t prow = kCache ? ((size_t)(b * T + t_row) * Hq + kvh * G + hg_row) : 0;
  float* const part = kCache ? a.partial + (prow * a.num_splits + split) * (D + 4) : nullptr;
  if constexpr (kCache) {
    if (a.num_splits > 1) {
      const int first = split * a.split_tiles;
      if (first >= ntiles) {
        if (row_ok && g == 0) part[D] = -INFINITY;
        return;
      }
      j_lo += first * kBN;
      ntiles = min(ntiles - first, a.split_tiles);
    }
  }

  const uint16_t* kbase = kr + (size_t)(b * Hkv + kvh) * T * D;
  const uint16_t* vbase = vp + ((size_t)b * T * Hkv + kvh) * D;
  const size_t vstride = (size_t)Hkv * D;
  const size_t cache_head = kCache ? (size_t)(b * Hkv + kvh) * a.cap * D : 0;

  // HBM -> LDS without registers: each wave moves PER_WAVE 1 KB pieces of
  // both tiles. Keys past the end read as zeros (without a cache) or re-read
  // the last key (in a chunk): finite values that the causal mask hides
  // (their probabilities are exactly 0). In a chunk, keys before p0 come
  // from the cache: slot j, or j mod cap in a ring.
  //
  // koff / voff are the byte offsets of this lane's pieces inside a tile, so
  // a whole tile (ending at or before the last key, wholly in the chunk or
  // wholly in consecutive cache slots) is a uniform base plus fixed lane
  // offsets. V's swizzle repeats every KPP keys (the keys of one piece), so
  // its pieces sit a fixed stride apart and one lane offset serves them all.
  constexpr int KPP = 64 / CH;  // keys per 1 KB piece
  uint32_t koff[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int P = 64 * (wave * PER_WAVE + i) + lane;
    const int key = P / CH, pos = P % CH;
    koff[i] = 2u * (uint32_t)(key * D + 8 * (pos ^ Swz<D>::k(key)));
  }
  const int key_l = wave * PER_WAVE * KPP + lane / CH;  // the lane's key in the wave's first piece
  const uint32_t vswz = 8 * ((lane % CH) ^ Swz<D>::v(key_l));
  const uint32_t voff = 2u * (__umul24(key_l, (unsigned)vstride) + vswz);
  // V in a cache has rows D apart (a chunk's V rows are Hkv D apart).
  const uint32_t vcoff = 2u * ((uint32_t)key_l * D + vswz);
  // Without a cache a tile is one descriptor pair ending at the sequence's
  // last key (loads past it return zeros and touch no memory), so the copy
  // has no branch; the bound is on the vector offset alone, so each V piece
  // carries its own offset.
  uint32_t voffs[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) voffs[i] = voff + (uint32_t)(i * KPP) * (uint32_t)vstride * 2u;
  // A full layer's prompt reads V^T rows (one per dim, t_pad slots) instead:
  // a 1 KB piece holds 8 dims x 64 slots; lane l copies dim 8 piece + l / 8,
  // and its 16 bytes land at chunk position l % 8, which holds source chunk
  // (l % 8) ^ SwzT(dim).
  constexpr bool VT = kCache == 0 && !SL && D == 128;
  uint32_t vtoffs[VT ? PER_WAVE : 1];
  if constexpr (VT) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int dim = 8 * (wave * PER_WAVE + i) + (lane >> 3);
      vtoffs[i] = 2u * ((uint32_t)dim * (uint32_t)a.t_pad + 8u * (uint32_t)((lane & 7) ^ SwzT::c(dim)));
    }
  }
  const uint16_t* vt_head = VT ? a.v_t + (size_t)(b * Hkv + kvh) * D * a.t_pad : nullptr;
  auto load_tile = [&](int j0, int st) {
    if constexpr (kCache == 2) {
      // cache slots j0.. of this sequence and KV head, rows D apart; the
      // descriptors end at the chunk's last key
      const int nk = min(kBN, j_last - j0 + 1);
      const size_t off = cache_head + (size_t)j0 * D;
      const __amdgpu_buffer_rsrc_t kres =
          tile_rsrc(static_cast<const uint16_t*>(a.k_cache) + off, (uint32_t)(nk * D * 2));
      const __amdgpu_buffer_rsrc_t vres =
          tile_rsrc(static_cast<const uint16_t*>(a.v_cache) + off, (uint32_t)(nk * D * 2));
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int I = wave * PER_WAVE + i;
        copy16_to_lds(kres, (lds_void_t*)&stg(st).k[512 * I], koff[i], 0u);
        copy16_to_lds(vres, (lds_void_t*)&stg(st).v[512 * I],
                      vcoff + (uint32_t)(i * KPP * D * 2), 0u);
      }
      return;
    }
    if constexpr (!kCache) {
      const int nk = min(kBN, j_last - j0 + 1);  // keys of the tile in the sequence, >= 1
      const __amdgpu_buffer_rsrc_t kres = tile_rsrc(kbase + (size_t)j0 * D, (uint32_t)(nk * D * 2));
      // (V^T: tiles start at multiples of 64, so a tile never runs past t_pad)
      const __amdgpu_buffer_rsrc_t vres =
          VT ? tile_rsrc(vt_head + j0, (uint32_t)((D * a.t_pad - j0) * 2))
             : tile_rsrc(vbase + (size_t)j0 * vstride, (uint32_t)(((nk - 1) * vstride + D) * 2));
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int I = wave * PER_WAVE + i;
        copy16_to_lds(kres, (lds_void_t*)&stg(st).k[512 * I], koff[i], 0u);
        copy16_to_lds(vres, (lds_void_t*)&stg(st).v[512 * I], VT ? vtoffs[VT ? i : 0] : voffs[i], 0u);
      }
      return;
    }
    const int kmax = j_last - j0;
    // a whole tile through buffer descriptors: uniform bases, the lane
    // offsets above, no vector arithmetic
    auto whole = [&](const void* kb, const void* vb, uint32_t vo, uint32_t vrow, uint32_t vbytes) {
      const __amdgpu_buffer_rsrc_t kres = tile_rsrc(kb, kBN * D * 2);
      const __amdgpu_buffer_rsrc_t vres = tile_rsrc(vb, vbytes);
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int I = wave * PER_WAVE + i;
        copy16_to_lds(kres, (lds_void_t*)&stg(st).k[512 * I], koff[i], 0u);
        copy16_to_lds(vres, (lds_void_t*)&stg(st).v[512 * I], vo, (uint32_t)i * KPP * vrow * 2);
      }
    };
    if (kmax >= kBN - 1 && j0 >= p0) {  // every key in this call's chunk
      whole(kbase + (size_t)(j0 - p0) * D, vbase + (size_t)(j0 - p0) * vstride, voff,
            (uint32_t)vstride, (uint32_t)(((kBN - 1) * vstride + D) * 2));
      return;
    }
    if constexpr (kCache) {
      // every key in the cache, in consecutive slots
      const int slot0 = a.ring ? j0 % a.cap : j0;
      if (j0 + kBN <= p0 && slot0 + kBN <= a.cap) {
        const size_t off = cache_head + (size_t)slot0 * D;
        whole(static_cast<const uint16_t*>(a.k_cache) + off,
              static_cast<const uint16_t*>(a.v_cache) + off, vcoff, D, kBN * D * 2);
        return;
      }
    }
    auto issue = [&](int I, const void* ksrc, const void* vsrc) {
      __builtin_amdgcn_global_load_lds(ksrc, (lds_void_t*)&stg(st).k[512 * I], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vsrc, (lds_void_t*)&stg(st).v[512 * I], 16, 0, 0);
    };
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int I = wave * PER_WAVE + i;
      const int P = 64 * I + lane;
      const int key = P / CH, pos = P % CH;
      const int kk = min(key, kmax);
      const int j = j0 + kk;
      if (kCache && j < p0) {
        const size_t off = cache_head + (size_t)(a.ring ? j % a.cap : j) * D;
        issue(I, static_cast<const uint16_t*>(a.k_cache) + off + 8 * (pos ^ Swz<D>::k(key)),
              static_cast<const uint16_t*>(a.v_cache) + off + 8 * (pos ^ Swz<D>::v(key)));
      } else {
        issue(I, kbase + (size_t)(j - p0) * D + 8 * (pos ^ Swz<D>::k(key)),
              vbase + (size_t)(j - p0) * vstride + 8 * (pos ^ Swz<D>::v(key)));
      }
    }
  };

  // ---- the block's Q rows go to stage 1 (idle until the loop starts) or,
  // with 8 waves, to the Q/output area; four whole rows per 1 KB piece. Chunk
  // c of row r sits at position c ^ swz(r), the layout K tiles use, so the
  // fragment reads below are conflict-free.
  {
    constexpr int Q_PIECES = kRows * D * 2 / 1024 / kWaves;
    uint16_t* qs = KW > 4 ? sm.qo : reinterpret_cast<uint16_t*>(&stage1);
#pragma unroll
    for (int i = 0; i < Q_PIECES; ++i) {
      const int I = wave * Q_PIECES + i;
      const int Pc = 64 * I + lane;
      const int r = Pc / CH, pos = Pc % CH;
      int dt, hg;
      split_local(min(r, nrows - 1), dt, hg);
      const uint16_t* src = qp + blk_row * D + (uint32_t)((__umul24(dt, Hq) + hg) * D + 8 * (pos ^ Swz<D>::k(r)));
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)&qs[512 * I], 16, 0, 0);
    }
  }

  // ---- cos/sin rows of the workgroup's positions go to LDS when they fit;
  // else Q reads them from the global table.
  const int half = a.rope.half, rdims = a.rope.rdims;
  const float2* cs_seq = a.cs_table + (size_t)b * a.cs_bstride;  // this sequence's rows
  const int cs_bytes = (t_hi - t_lo + 1) * half * 8;
  const bool cs_lds = half > 0 && cs_bytes <= (int)sizeof(sm.cs);
  if (cs_lds) {
    const char* src0 = reinterpret_cast<const char*>(cs_seq + (size_t)t_lo * half);
    const int nblk = (cs_bytes + 1023) / 1024;
    for (int I = wave; I < nblk; I += kWaves) {
      const int off = min(1024 * I + 16 * lane, cs_bytes - 16);
      __builtin_amdgcn_global_load_lds((const void*)(src0 + off),
                                       (lds_void_t*)(reinterpret_cast<char*>(sm.cs) + 1024 * I),
                                       16, 0, 0);
    }
  }

  // The gate logit is needed only at the end; fetch it now so its latency
  // hides behind the tile loop.
  const float gate_logit =
      bf16_to_f32(static_cast<const uint16_t*>(a.gate)[blk_row + (uint32_t)(__umul24(dt_row, Hq) + hg_row)]);

  // Tile 0 moves while Q is rotated. Vector-memory counts retire in issue
  // order, so waiting until this wave's 2 PER_WAVE tile-0 pieces are the only
  // ones left means its Q and cos/sin pieces have landed. (ntiles >= 1: the
  // diagonal key is always visible.)
  load_tile(j_lo, 0);
  __builtin_amdgcn_s_waitcnt((2 * PER_WAVE) | (7 << 4) | (15 << 8));  // vmcnt(2 PER_WAVE)
  __builtin_amdgcn_s_barrier();  // every wave's Q and cos/sin pieces have landed

  // ---- Q^T fragments: lane holds row n, dims 16s+8g..+7, rotated below.
  const uint16_t* qrow = qp + blk_row * D + (uint32_t)((__umul24(dt_row, Hq) + hg_row) * D);
  u32x4_t qraw[NS];
  {
    const int r = wave * kRowsPerWave + n;
    const uint16_t* qs = (KW > 4 ? sm.qo : reinterpret_cast<const uint16_t*>(&stage1)) + r * D;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qraw[s] = *reinterpret_cast<const u32x4_t*>(qs + 8 * ((2 * s + g) ^ Swz<D>::k(r)));
  }

  // q is rotated and multiplied by scale * log2(e) before its one rounding to
  // bf16, so scores come out of the MFMA in log2 units.
  const float sc = a.scale * kLog2e;
  bf16x8_t qf[NS];
  if (half == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float x[8];
      unpack8(qraw[s], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= sc;
      qf[s] = pack8(x);
    }
  } else if (half % 16 == 0) {
    // The RoPE partner of every chunk sits in this lane, half/16 chunks away.
    const float2* csl = sm.cs + dt_row * half;
    const float2* csg = cs_seq + (size_t)t_row * half;
    switch (half / 16) {
#define HGQA_ROPE_CASE(H)                                 \
  case H:                                                 \
    if (cs_lds) rope_q_inlane<NS, H>(qraw, qf, g, csl, sc);   \
    else rope_q_inlane<NS, H>(qraw, qf, g, csg, sc);          \
    break;
      HGQA_ROPE_CASE(1)
      HGQA_ROPE_CASE(2)
      HGQA_ROPE_CASE(3)
      HGQA_ROPE_CASE(4)
#undef HGQA_ROPE_CASE
    }
  } else {
    // r/2 an odd multiple of 8: partner chunks are read again from HBM.
    const float2* csrow = cs_seq + (size_t)t_row * half;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d0 = 16 * s + 8 * g;
      float x[8];
      unpack8(qraw[s], x);
      if (d0 < rdims) {
        const bool first = d0 < half;
        const int i0 = first ? d0 : d0 - half;
        u32x4_t praw = *reinterpret_cast<const u32x4_t*>(qrow + (first ? d0 + half : d0 - half));
        rotate8(x, praw, csrow + i0, first ? -1.0f : 1.0f);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= sc;
      qf[s] = pack8(x);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // tile 0 has landed; Q and the cos/sin rows are read before stage 1 is refilled

  f32x16_t O[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) O[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;
  // Scores are kept relative to m_use (m_run, or 0 while a row has seen no
  // key) in log2 units: q carries scale * log2(e), and the score products
  // start from -m_use instead of zero, so the exponent needs no arithmetic.
  float m_use = 0.0f;
  f32x16_t negm = {};
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // V^T operand supplier addresses for ds_read_b64_tr_b16: lane r of each
  // 16-lane group points at key (4g + r/4) and dims 4(r%4).. of its d half.
  const int r16 = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  const int vkey0 = 4 * g + (r16 >> 2);
  const int vd = 16 * dhalf + 4 * (r16 & 3);


  // One K/V tile. NKB counts the 32-key halves computed: the upper half of a
  // wave's last tile often holds only keys past all its rows, and is skipped.
  // LOAD: the next tile is copied into the other stage during this one.
  // STAGE: the stage this tile sits in, known at compile time.
  auto tile = [&](int it, auto nkb_tag, auto first_tag, auto load_tag, auto stage_tag) {
    constexpr int NKB = decltype(nkb_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    constexpr bool LOAD = decltype(load_tag)::value;
    constexpr int st = decltype(stage_tag)::value;
    const int j0 = j_lo + it * kBN;
    // A chunk over the cache and its own keys branches (chunk or cache, ring
    // wrap): issue it first.
    if constexpr (kCache == 1 && LOAD) load_tile(j0 + kBN, st ^ 1);
    if (kCache && !wave_rows) {
      // a chunk of a few tokens leaves whole waves without rows: they only
      // copy their share of the tiles (no products, no LDS fragment reads)
      // (the empty asm keeps the compiler from hoisting this copy, identical
      // to the one in the products' schedule below, above the branch)
      asm volatile("" ::: "memory");
      if constexpr (kCache == 2 && LOAD) load_tile(j0 + kBN, st ^ 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      return;
    }
    const uint16_t* ks = stg(st).k;
    const uint16_t* vs = stg(st).v;

    // S^T for two 32-key blocks, the blocks' products alternating; each K
    // fragment read runs RA products ahead of its product, so the LDS
    // latency hides behind the products in between
    f32x16_t S[2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) S[kb] = FIRST ? f32x16_t{} : negm;
    // Otherwise the copy has no branch and joins the products' schedule.
    if constexpr (kCache != 1 && LOAD) load_tile(j0 + kBN, st ^ 1);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int key = 32 * kb + n;
        const int pos = (2 * s + g) ^ Swz<D>::k(key);
        bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(ks + key * D + 8 * pos);
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], S[kb], 0, 0, 0);
      }
    {
      // The next tile's copy pieces go one after every second product. Issued
      // together at the top of the tile, every wave of the CU queued on the
      // copy path at once and no products ran meanwhile.
      constexpr int NM = NS * NKB, RA = 4 < NM ? 4 : NM;
      constexpr int NC = (kCache != 1 && LOAD) ? 2 * PER_WAVE : 0;
      static_assert(NC == 0 || 2 * NC <= NM, "a copy piece after every second product");
      __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);  // the first RA fragment reads
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a product
        if (i + RA < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a read RA ahead
        if (i % 2 == 1 && i / 2 < NC) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // a copy
      }
    }

    // mask only where the tile crosses the diagonal or the window edge
    const bool need_mask = (j0 + kBN - 1 > tw_lo) || (SL && j0 < tw_hi - a.window + 1);
    if (need_mask) {
      // key j = j0 + 4g + off is visible iff 0 <= t_row - j < W (W = 2^31 when
      // full): one unsigned compare per element against a per-lane base.
      const int base = t_abs - j0 - 4 * g;
      const unsigned wlim = SL ? (unsigned)a.window : 0x80000000u;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = 32 * kb + 8 * (v >> 2) + (v & 3);
          S[kb][v] = ((unsigned)(base - off) < wlim) ? S[kb][v] : -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // m_run is a per-row reference, not the exact running maximum: it moves
    // only when a score exceeds it by more than 2^8, so probabilities stay
    // below 256 and the output is rescaled rarely; O / l is exact for any
    // reference. S already holds score - m_use in log2 units (the first tile
    // holds plain scores); when the reference moves, S shifts with it.
    const float m_cand = FIRST ? mx : mx + m_use;
    const bool need = m_cand > m_run + 8.0f;
    if (FIRST || __any(need)) {
      if (!FIRST) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_cand) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i) O[i] *= alpha;
      }
      const float shift = need ? m_cand - (FIRST ? 0.0f : m_use) : 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) S[kb] -= shift;
      m_run = need ? m_cand : m_run;
      m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      negm = f32x16_t{} - m_use;
    }

    // P = exp2(S), packed to bf16 in the B-operand order of PV; the row sum
    // is taken over the same rounded values.
    u32x4_t pk[4];
#pragma unroll
    for (int ks4 = 0; ks4 < 2 * NKB; ++ks4) {
      const int kb = ks4 >> 1, hh = ks4 & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pa = __builtin_amdgcn_exp2f(S[kb][8 * hh + 2 * e]);
        const float pb = __builtin_amdgcn_exp2f(S[kb][8 * hh + 2 * e + 1]);
        const bf16x2_t pv = {(__bf16)pa, (__bf16)pb};
        pk[ks4][e] = __builtin_bit_cast(uint32_t, pv);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pv, ones, l_run, false);
      }
    }

    // O^T += V^T P^T, 4 k-steps of 16 keys; V^T comes transposed out of LDS
    // (or, from a V^T tile, straight: lane l reads dim l % 32 of the block,
    // chunk 2 ks4 + l / 32, the eight keys P's lane holds for that k-half).
#pragma unroll
    for (int ks4 = 0; ks4 < 2 * NKB; ++ks4) {
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk[ks4]);
      const int k0 = 16 * ks4 + vkey0, k1 = k0 + 8;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i16x8_t va;
        if constexpr (VT) {
          const int dim = 32 * db + n, c = 2 * ks4 + g;
          va = *reinterpret_cast<const i16x8_t*>(vs + dim * kBN + 8 * (c ^ SwzT::c(dim)));
        } else {
          const int d = 32 * db + vd;
          const int c = d >> 3, hw = d & 7;
          const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(vs + k0 * D + 8 * (c ^ Swz<D>::v(k0)) + hw));
          const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(vs + k1 * D + 8 * (c ^ Swz<D>::v(k1)) + hw));
          va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va), pb,
                                                         O[db], 0, 0, 0);
      }
    }

    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of the next tile has landed
    __syncthreads();
  };

  // The first tile (when it is not also the last) is its own copy: it sets
  // the softmax reference without rescaling the still-zero output.
  using Later = std::integral_constant<bool, false>;
  using First = std::integral_constant<bool, true>;
  using Full = std::integral_constant<int, 2>;
  using Half = std::integral_constant<int, 1>;
  using Load = std::integral_constant<bool, true>;
  using NoLoad = std::integral_constant<bool, false>;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // Unrolled by two, so that every copy of the tile body names its stages
  // as distinct LDS objects: the compiler then lets the next tile's copies
  // move among this tile's fragment reads, and waits for them only where a
  // read could touch the stage being filled.
  if (ntiles > 1) tile(0, Full{}, First{}, Load{}, S0{});
  for (int it = 1; it + 1 < ntiles; it += 2) {
    tile(it, Full{}, Later{}, Load{}, S1{});
    if (it + 2 < ntiles) tile(it + 1, Full{}, Later{}, Load{}, S0{});
  }
  const bool last_half = j_lo + (ntiles - 1) * kBN + 32 > tw_hi;
  if ((ntiles - 1) & 1) {
    if (last_half) tile(ntiles - 1, Half{}, Later{}, NoLoad{}, S1{});
    else tile(ntiles - 1, Full{}, Later{}, NoLoad{}, S1{});
  } else {
    if (last_half) tile(ntiles - 1, Half{}, Later{}, NoLoad{}, S0{});
    else tile(ntiles - 1, Full{}, Later{}, NoLoad{}, S0{});
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if constexpr (kCache) {
    if (a.num_splits > 1) {
      // partial of this split: the unnormalised output and the sum relative
      // to the reference (log2 units), which is -inf when the row saw no key
      if (row_ok) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4_t*>(part + 32 * db + 8 * q4 + 4 * g) =
                f32x4_t{O[db][4 * q4], O[db][4 * q4 + 1], O[db][4 * q4 + 2], O[db][4 * q4 + 3]};
        if (g == 0) *reinterpret_cast<float2*>(part + D) = make_float2(m_run, l_tot);
      }
      return;
    }
  }

  // ---- epilogue: normalise and gate in registers, then turn the O^T
  // fragments into row-major rows in LDS (stage 0, idle because the loop
  // ended on a barrier with no load in flight, or with 8 waves the Q/output
  // area) so that the stores write whole rows.
  const float inv = row_ok ? sigmoidf_dev(gate_logit) / l_tot : 0.0f;
  uint16_t* ow = (KW > 4 ? sm.qo : reinterpret_cast<uint16_t*>(&stage0)) + wave * (kRowsPerWave * D);  // this wave's rows
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c = 4 * db + q4;  // 16-byte chunk of dims 32 db + 8 q4 ..
      u32x2_t w = {pack_bf16x2(O[db][4 * q4] * inv, O[db][4 * q4 + 1] * inv),
                   pack_bf16x2(O[db][4 * q4 + 2] * inv, O[db][4 * q4 + 3] * inv)};
      *reinterpret_cast<u32x2_t*>(ow + n * D + 8 * (c ^ Swz<D>::k(n)) + 4 * g) = w;
    }
  __syncthreads();
  constexpr int O_PIECES = kRowsPerWave * D * 2 / 1024;
  uint16_t* op = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int i = 0; i < O_PIECES; ++i) {
    const int Pc = 64 * i + lane;
    const int r = Pc / CH, pos = Pc % CH;  // row of the wave, LDS position
    const int rb_local = wave * kRowsPerWave + r;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ow + r * D + 8 * pos);
    int dt, hg;
    split_local(rb_local, dt, hg);
    if (rb_local < nrows)
      *reinterpret_cast<u32x4_t*>(op + blk_row * D + (uint32_t)((__umul24(dt, Hq) + hg) * D + 8 * (pos ^ Swz<D>::k(r)))) = v;
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
  const float2* cs = a.cs_table + (size_t)b * a.cs_bstride + (size_t)t * half;
  for (int d = lane; d < D; d += 64) {
    float x = q[d];
    if (d < half) x = fmaf(x, cs[d].x, -q[d + half] * cs[d].y);
    else if (d < rdims) x = fmaf(x, cs[d - half].x, q[d - half] * cs[d - half].y);
    qs[d] = x;
  }
  __syncthreads();
  // Absolute positions: row t sits at p0 + t; keys before p0 (a chunk that
  // continues a cached sequence) come from the cache, slot j or j mod cap.
  const int p0 = prefill_p0(a, b), ta = p0 + t;
  const int lo = a.sliding ? max(0, ta - a.window + 1) : 0;
  const float* kr = static_cast<const float*>(a.k_rot) + (size_t)(b * a.Hkv + kvh) * T * D;
  const float* v = static_cast<const float*>(a.v) + ((size_t)b * T * a.Hkv + kvh) * D;
  const size_t vstride = (size_t)a.Hkv * D;
  const size_t cache_head = (size_t)(b * a.Hkv + kvh) * a.cap * D;
  auto key_row = [&](int j) -> const float* {
    if (j < p0) return static_cast<const float*>(a.k_cache) + cache_head + (size_t)(a.ring ? j % a.cap : j) * D;
    return kr + (size_t)(j - p0) * D;
  };
  auto value_row = [&](int j) -> const float* {
    if (j < p0) return static_cast<const float*>(a.v_cache) + cache_head + (size_t)(a.ring ? j % a.cap : j) * D;
    return v + (size_t)(j - p0) * vstride;
  };
  float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int j0 = lo; j0 <= ta; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j <= ta) {
      const float* krow = key_row(j);
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], krow[d], dot);
      s = dot * a.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = expf(m - mn);
    const float p = (j <= ta) ? expf(s - mn) : 0.0f;
    l = l * alpha + wave_sum(p);
    ps[lane] = p;
    __syncthreads();
    o0 *= alpha;
    o1 *= alpha;
    const int nk = min(64, ta - j0 + 1);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = ps[jj];
      const float* vrow = value_row(j0 + jj);
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

// Log-sum-exp merge of a chunk's key splits, then the gate. One block per
// (sequence, row, head) of D/4 x NG threads: thread t takes dims 4 (t % (D/4))
// .. + 3 and every NG-th split from t / (D/4); the NG split groups then add
// up through LDS, so a call with many splits (one sequence's verify step
// over a long context) is not one long dependent chain per thread. Splits
// whose rows saw no key (reference -inf) carry no weight; every row sees at
// least its own position, so some split has a finite reference.
constexpr int kPMergeMaxThreads = 256;
__global__ __launch_bounds__(kPMergeMaxThreads) void prefill_merge_kernel(PrefillArgs a) {
  __shared__ float wave_max[kPMergeMaxThreads / 64];
  __shared__ f32x4_t gacc[kPMergeMaxThreads];
  __shared__ float gsum[kPMergeMaxThreads];
  const size_t row = blockIdx.x;  // (b T + t) Hq + h
  const int D = a.D, ns = a.num_splits, rec = D + 4;  // record: D outputs, reference, sum, 2 spare
  const int tid = threadIdx.x, nt = blockDim.x, DQ = D / 4, ng = nt / DQ;
  const float* pr = a.partial + row * ns * rec;

  float M = -INFINITY;
  for (int s = tid; s < ns; s += nt) M = fmaxf(M, pr[(size_t)s * rec + D]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if ((tid & 63) == 0) wave_max[tid >> 6] = M;
  __syncthreads();
  M = wave_max[0];
  for (int w = 1; w < nt / 64; ++w) M = fmaxf(M, wave_max[w]);

  const int dq = tid % DQ, grp = tid / DQ;
  f32x4_t acc = {};
  float l = 0.0f;
  for (int s = grp; s < ns; s += ng) {
    const float* p = pr + (size_t)s * rec;
    const float2 ml = *reinterpret_cast<const float2*>(p + D);
    if (ml.x == -INFINITY) continue;
    const float f = __builtin_amdgcn_exp2f(ml.x - M);
    acc += f * *reinterpret_cast<const f32x4_t*>(p + 4 * dq);
    l = fmaf(ml.y, f, l);
  }
  gacc[tid] = acc;
  gsum[tid] = l;
  __syncthreads();
  if (tid < DQ) {
    f32x4_t r = gacc[tid];
    float lt = gsum[tid];
    for (int g = 1; g < ng; ++g) {
      r += gacc[g * DQ + tid];
      lt += gsum[g * DQ + tid];
    }
    const float gs = sigmoidf_dev(bf16_to_f32(static_cast<const uint16_t*>(a.gate)[row])) / lt;
    const u32x2_t w = {pack_bf16x2(gs * r[0], gs * r[1]), pack_bf16x2(gs * r[2], gs * r[3])};
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + row * D + 4 * tid) = w;
  }
}

// Threads of a merge block: D/4 per split group, at least one wave, and
// groups up to the split count (at most 256 threads).
static int prefill_merge_threads(int num_splits, int D) {
  const int dq = D / 4;
  int ng = 64 / dq;
  while (ng * dq < kPMergeMaxThreads && ng < num_splits) ng *= 2;
  return ng * dq;
}

// Waves per workgroup. 8 (one workgroup per CU, each K/V tile copied once
// for 256 rows) when a block visits many tiles: full layers and windows of
// 1024 keys or more (measured: full layers 4-5% faster, W = 2048 3-4%). 4
// for short windows, where a workgroup's fixed costs weigh more and two
// workgroups per CU hide them (W = 512: 8 waves is 9% slower), and for
// chunks of fewer than 2048 rows (a few new tokens would leave most of 256
// rows empty). D = 128 only; a.waves (4 or 8) overrides the choice.
static int prefill_waves(const PrefillArgs& a) {
  if (a.D != 128) return 4;
  if (a.waves == 4 || a.waves == 8) return a.waves;
  const bool long_span = !a.sliding || a.window >= 1024;
  const bool enough_rows = a.k_cache == nullptr || (long long)a.T * a.G >= 2048;
  return long_span && enough_rows ? 8 : 4;
}

template <int D, int kCache, int KW>
static void launch_bf16(const PrefillArgs& a, dim3 grid, hipStream_t s) {
  if (a.sliding)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, kCache, KW, true>), grid, dim3(KW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<D, kCache, KW, false>), grid, dim3(KW * 64), 0, s, a);
}

// Chunk calls whose grid would not fill the chip twice over (few rows, few
// sequences) split each block's key range, at least kMinSplitTiles tiles per
// split, aiming at kSplitTargetBlocks workgroups; bf16 only.
constexpr int kMinSplitTiles = 16;
constexpr int kSplitTargetBlocks = 2048;

size_t plan_prefill_splits(PrefillArgs& a, Elem e, int max_end_pos, int split_tiles_override) {
  a.num_splits = 1;
  a.split_tiles = 0;
  if (e != Elem::BF16 || a.k_cache == nullptr || a.B == 0 || a.T == 0) return 0;
  const int kw = prefill_waves(a);
  const long long nrb = ((long long)a.T * a.G + kw * kRowsPerWave - 1) / (kw * kRowsPerWave);
  const long long blocks = nrb * a.B * a.Hkv;
  // longest key range of a block: the whole context (full) or the window
  // plus the block's positions (sliding)
  const long long span = a.sliding ? std::min<long long>(max_end_pos, (long long)a.window + a.T)
                                   : max_end_pos;
  const long long tiles = span / kBN + 2;
  long long st;
  if (split_tiles_override > 0) {
    st = split_tiles_override;
  } else {
    if (blocks * kw >= 2LL * 256 * 8) return 0;
    long long ns = (kSplitTargetBlocks + blocks - 1) / blocks;
    ns = std::min(ns, tiles / kMinSplitTiles);
    if (ns <= 1) return 0;
    st = (tiles + ns - 1) / ns;
  }
  const long long ns = (tiles + st - 1) / st;
  if (ns <= 1) return 0;
  a.num_splits = (int)ns;
  a.split_tiles = (int)st;
  return (size_t)a.B * a.T * a.Hq * ns * (a.D + 4) * sizeof(float);
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
  const bool cache = a.k_cache != nullptr;
  const int kw = prefill_waves(a);
  const long long rows = (long long)kw * kRowsPerWave;
  const long long blocks = (TG + rows - 1) / rows * a.B * a.Hkv * (cache ? a.num_splits : 1);
  const dim3 grid((unsigned)blocks);
  if (a.D == 128 && cache && a.keys_in_cache) {  // full layers only
    if (kw == 8)
      hipLaunchKernelGGL((prefill_bf16_kernel<128, 2, 8, false>), grid, dim3(8 * 64), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<128, 2, 4, false>), grid, dim3(4 * 64), 0, s, a);
  } else if (a.D == 128) {
    if (cache && kw == 8) launch_bf16<128, 1, 8>(a, grid, s);
    else if (cache) launch_bf16<128, 1, 4>(a, grid, s);
    else if (kw == 8) launch_bf16<128, 0, 8>(a, grid, s);
    else launch_bf16<128, 0, 4>(a, grid, s);
  } else {
    if (cache) launch_bf16<64, 1, 4>(a, grid, s);
    else launch_bf16<64, 0, 4>(a, grid, s);
  }
  err = hipGetLastError();
  if (err != hipSuccess || !cache || a.num_splits <= 1) return err;
  hipLaunchKernelGGL(prefill_merge_kernel, dim3((unsigned)((long long)a.B * a.T * a.Hq)),
                     dim3(prefill_merge_threads(a.num_splits, a.D)), 0, s, a);
  return hipGetLastError();
}

}  // namespace hgqa
