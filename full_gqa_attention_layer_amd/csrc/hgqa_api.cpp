// C-ABI front end of libhgqa.so: argument checks, RoPE frequency set-up and
// dispatch to the gfx950 kernels. Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/hgqa.h"
#include "hgqa_internal.h"

namespace {

thread_local std::string g_last_error;

// hgqa_set_tuning overrides (0: the library's own choice).
std::atomic<int> g_prefill_waves{0};
std::atomic<int> g_decode_split_keys{0};
std::atomic<int> g_chunk_split_tiles{0};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return HGQA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct Layer {
  int sliding, window, Hq, G, Hkv, D, rdims, half;
  float theta, scale;
  // llama3 frequency scaling (full layers); factor <= 1: none
  double scale_factor, low_freq, high_freq, original_positions;
  hgqa::Elem elem;
  size_t esize;
};

// Validates a layer descriptor; fills `out`. Returns HGQA_OK or an error.
int check_layer(const hgqa_layer* L, Layer* out) {
  if (!L) return fail(HGQA_EINVAL, "layer descriptor is NULL");
  if (L->layer_type != HGQA_FULL && L->layer_type != HGQA_SLIDING)
    return fail(HGQA_EINVAL, "layer_type %d is neither HGQA_FULL nor HGQA_SLIDING", L->layer_type);
  if (L->layer_type == HGQA_SLIDING && L->window < 1)
    return fail(HGQA_EINVAL, "a sliding layer needs window >= 1 (got %d)", L->window);
  if (L->num_q_heads < 1) return fail(HGQA_EINVAL, "num_q_heads must be >= 1");
  if (L->gqa_ratio < 1) return fail(HGQA_EINVAL, "gqa_ratio must be >= 1");
  if (L->num_q_heads % L->gqa_ratio)
    return fail(HGQA_EINVAL, "num_q_heads %d is not a multiple of gqa_ratio %d", L->num_q_heads,
                L->gqa_ratio);
  if (L->dtype != HGQA_BF16 && L->dtype != HGQA_FP32)
    return fail(HGQA_EINVAL, "dtype %d is neither HGQA_BF16 nor HGQA_FP32", L->dtype);
  if (L->head_dim != 64 && L->head_dim != 128)
    return fail(HGQA_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", L->head_dim);
  if (!std::isfinite(L->rope_theta) || L->rope_theta < 0.0f)
    return fail(HGQA_EINVAL, "rope_theta must be finite and >= 0");
  if (!std::isfinite(L->rotary_fraction) || L->rotary_fraction < 0.0f || L->rotary_fraction > 1.0f)
    return fail(HGQA_EINVAL, "rotary_fraction must lie in [0, 1]");
  if (!std::isfinite(L->softmax_scale)) return fail(HGQA_EINVAL, "softmax_scale is not finite");
  Layer& o = *out;
  o.sliding = L->layer_type == HGQA_SLIDING;
  o.window = o.sliding ? L->window : 0;
  o.Hq = L->num_q_heads;
  o.G = L->gqa_ratio;
  o.Hkv = o.Hq / o.G;
  o.D = L->head_dim;
  o.theta = L->rope_theta;
  o.elem = L->dtype == HGQA_BF16 ? hgqa::Elem::BF16 : hgqa::Elem::F32;
  o.esize = L->dtype == HGQA_BF16 ? 2 : 4;
  int r = (int)std::lround((double)L->rotary_fraction * o.D);
  if (o.theta == 0.0f) r = 0;
  if (r % 2) return fail(HGQA_EINVAL, "rotary dims round(f*D) = %d must be even", r);
  if (o.elem == hgqa::Elem::BF16 && r % 16)
    return fail(HGQA_EUNSUPPORTED, "bf16 layers need rotary dims %% 16 == 0 (got %d)", r);
  o.rdims = r;
  o.half = r / 2;
  o.scale = L->softmax_scale > 0.0f ? L->softmax_scale : (float)(1.0 / std::sqrt((double)o.D));
  if (!std::isfinite(L->rope_scaling_factor) || !std::isfinite(L->rope_low_freq_factor) ||
      !std::isfinite(L->rope_high_freq_factor))
    return fail(HGQA_EINVAL, "rope scaling parameters must be finite");
  // Only full layers carry the scaling; sliding layers keep the plain RoPE.
  o.scale_factor = (!o.sliding && L->rope_scaling_factor > 1.0f) ? L->rope_scaling_factor : 1.0;
  o.low_freq = L->rope_low_freq_factor > 0.0f ? L->rope_low_freq_factor : 1.0;
  o.high_freq = L->rope_high_freq_factor > 0.0f ? L->rope_high_freq_factor : 4.0;
  o.original_positions = L->rope_original_max_positions > 0 ? L->rope_original_max_positions : 131072.0;
  if (o.scale_factor > 1.0 && !(o.high_freq > o.low_freq))
    return fail(HGQA_EINVAL, "rope_high_freq_factor (%g) must exceed rope_low_freq_factor (%g)",
                o.high_freq, o.low_freq);
  return HGQA_OK;
}

// Frequency w of a RoPE pair after the llama3 long-context rescaling: short
// wavelengths keep w, long ones get w / factor, a linear blend in between.
double llama3_frequency(const Layer& l, double w) {
  const double wavelength = 2.0 * M_PI / w;
  if (wavelength < l.original_positions / l.high_freq) return w;
  if (wavelength > l.original_positions / l.low_freq) return w / l.scale_factor;
  const double s = (l.original_positions / wavelength - l.low_freq) / (l.high_freq - l.low_freq);
  return (1.0 - s) * w / l.scale_factor + s * w;
}

void fill_rope(const Layer& l, hgqa::RopeArgs* r) {
  std::memset(r, 0, sizeof *r);
  r->half = l.half;
  r->rdims = l.rdims;
  for (int i = 0; i < l.half; ++i) {
    double w = std::pow((double)l.theta, -2.0 * i / l.rdims);
    if (l.scale_factor > 1.0) w = llama3_frequency(l, w);
    r->freq_over_pi[i] = w / M_PI;
  }
}

// Largest element count any one buffer may hold; keeps 64-bit offsets exact
// and block counts within the grid limit.
constexpr long long kMaxElems = 1LL << 40;

// Rotated K [B,Hkv,T,D], then the cos/sin table: [T, r/2] shared by every
// sequence of a prompt at positions 0.., or [B, T, r/2] for chunks whose
// sequences start at their own positions.
size_t rotated_k_bytes(const Layer& l, int B, int T) {
  return round256((size_t)B * l.Hkv * T * l.D * l.esize);
}
int t_pad(int T) { return (T + 63) / 64 * 64; }
// V^T for full bf16 layers with D = 128, while one head's V^T rows stay
// within the 32-bit byte offsets of a buffer descriptor
bool uses_vt(const Layer& l, int T) {
  return !l.sliding && l.elem == hgqa::Elem::BF16 && l.D == 128 &&
         (long long)l.D * t_pad(T) * 2 < (1LL << 31);
}
size_t table_bytes(const Layer& l, int T) { return round256((size_t)T * l.half * sizeof(float2)); }
size_t vt_bytes(const Layer& l, int B, int T) {
  return uses_vt(l, T) ? round256((size_t)B * l.Hkv * l.D * t_pad(T) * sizeof(uint16_t)) : 0;
}
size_t prefill_ws(const Layer& l, int B, int T) {
  return rotated_k_bytes(l, B, T) + table_bytes(l, T) + vt_bytes(l, B, T);
}
size_t chunk_ws(const Layer& l, int B, int T) {
  return rotated_k_bytes(l, B, T) + round256((size_t)B * T * l.half * sizeof(float2));
}

// The key-split plan of a chunk call (the same for the workspace query and
// the call): fills a's split fields, returns the partial bytes (256-rounded).
size_t plan_splits(const Layer& l, hgqa::PrefillArgs& a, int max_end_pos) {
  a.k_cache = reinterpret_cast<const void*>(16);  // a chunk: the plan only tests for a cache
  a.sliding = l.sliding;
  a.window = l.window;
  // The merge launches one block per row: no splits past the grid limit
  // (reachable only through the split-tile override).
  if ((long long)a.B * a.T * a.Hq > 0x7fffffffLL) {
    a.num_splits = 1;
    a.split_tiles = 0;
    return 0;
  }
  return round256(hgqa::plan_prefill_splits(a, l.elem, max_end_pos,
                                            g_chunk_split_tiles.load(std::memory_order_relaxed)));
}

// Checks shared by the prefill entry points; n = tokens in this call, need =
// the workspace bytes the call needs.
int check_prefill_call(const Layer& l, int batch, int n, const void* q, const void* k,
                       const void* v, const void* gate, const void* out, const void* workspace,
                       size_t workspace_bytes, size_t need) {
  if (batch > 65535) return fail(HGQA_EUNSUPPORTED, "batch %d exceeds 65535", batch);
  if ((long long)batch * n * l.Hq * l.D > kMaxElems)
    return fail(HGQA_EUNSUPPORTED, "problem too large");
  const long long TG = (long long)n * l.G;
  if (l.elem == hgqa::Elem::BF16 && (TG + 127) / 128 * batch * l.Hkv > 0x7fffffffLL)
    return fail(HGQA_EUNSUPPORTED, "too many query blocks");
  if (!q || !k || !v || !gate || !out || !workspace)
    return fail(HGQA_EINVAL, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return fail(HGQA_EINVAL, "q, k, v, out and workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(HGQA_ENOSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if (out == q || out == k || out == v || out == gate)
    return fail(HGQA_EINVAL, "out must not alias an input");
  return HGQA_OK;
}

hgqa::PrefillArgs prefill_args(const Layer& l, int batch, int n, const void* q, const void* k,
                               const void* v, const void* gate, void* out, void* workspace) {
  hgqa::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate;
  a.out = out;
  a.k_rot = workspace;
  a.cs_table = reinterpret_cast<float2*>(static_cast<char*>(workspace) + rotated_k_bytes(l, batch, n));
  a.cs_bstride = 0;
  a.start_pos = nullptr;
  a.max_end_pos = n;
  a.waves = g_prefill_waves.load(std::memory_order_relaxed);
  a.num_splits = 1;
  a.split_tiles = 0;
  a.partial = nullptr;
  a.B = batch;
  a.T = n;
  a.Hq = l.Hq;
  a.Hkv = l.Hkv;
  a.G = l.G;
  a.D = l.D;
  a.sliding = l.sliding;
  a.window = l.window;
  a.scale = l.scale;
  fill_rope(l, &a.rope);
  return a;
}

// Partial bytes of a chunk call's key splits (0 without splits).
size_t split_ws(const Layer& l, int B, int n, int max_end_pos) {
  hgqa::PrefillArgs a{};
  a.B = B;
  a.T = n;
  a.Hq = l.Hq;
  a.Hkv = l.Hkv;
  a.G = l.G;
  a.D = l.D;
  a.waves = g_prefill_waves.load(std::memory_order_relaxed);
  return plan_splits(l, a, max_end_pos);
}

}  // namespace

int hgqa::decode_call(const void* layer_ptr, int batch, const void* q, const void* gate,
                      const void* k_cache, const void* v_cache, int cache_capacity,
                      const int32_t* seq_lens, int max_seq_len, void* workspace,
                      size_t workspace_bytes, void* out, void* stream, ScratchFn scratch_fn,
                      size_t scratch_bytes) {
  const hgqa_layer* layer = static_cast<const hgqa_layer*>(layer_ptr);
  Layer l;
  int rc = check_layer(layer, &l);
  if (rc != HGQA_OK) return rc;
  if (batch < 0) return fail(HGQA_EINVAL, "batch must be >= 0");
  if (batch == 0) return ok();
  if (batch > 65535) return fail(HGQA_EUNSUPPORTED, "batch %d exceeds 65535", batch);
  if (max_seq_len < 1) return fail(HGQA_EINVAL, "max_seq_len must be >= 1");
  if (cache_capacity < 1) return fail(HGQA_EINVAL, "cache_capacity must be >= 1");
  if (l.sliding && cache_capacity != l.window)
    return fail(HGQA_EINVAL, "a sliding layer's ring must hold exactly W = %d slots (got %d)",
                l.window, cache_capacity);
  if (!l.sliding && max_seq_len > cache_capacity)
    return fail(HGQA_ENOSPACE, "max_seq_len %d exceeds the full cache capacity %d", max_seq_len,
                cache_capacity);
  if (l.elem == hgqa::Elem::BF16 && l.G > 16)
    return fail(HGQA_EUNSUPPORTED, "bf16 decode supports gqa_ratio <= 16 (got %d)", l.G);
  if ((long long)batch * l.Hkv * cache_capacity * l.D > kMaxElems)
    return fail(HGQA_EUNSUPPORTED, "cache too large");
  if (!q || !gate || !k_cache || !v_cache || !seq_lens || !out)
    return fail(HGQA_EINVAL, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(HGQA_EINVAL, "q, the caches and out must be 16-byte aligned");
  if (out == q || out == gate) return fail(HGQA_EINVAL, "out must not alias an input");
  const hgqa::DecodePlan plan =
      hgqa::plan_decode(l.elem, batch, l.Hq, l.Hkv, l.D, l.sliding, l.window, max_seq_len,
                        g_decode_split_keys.load(std::memory_order_relaxed));
  if (scratch_fn && plan.workspace_bytes > 0) {
    if (plan.workspace_bytes > scratch_bytes)
      return fail(HGQA_ENOSPACE,
                  "this decode needs %zu bytes of split partials; the library's static scratch "
                  "holds %zu (use attn_decode with a workspace)",
                  plan.workspace_bytes, scratch_bytes);
    hipError_t e = scratch_fn(static_cast<hipStream_t>(stream), &workspace);
    if (e != hipSuccess)
      return fail(HGQA_EHIP, "decode scratch set-up failed: %s", hipGetErrorString(e));
    workspace_bytes = scratch_bytes;
  }
  if (plan.workspace_bytes > 0) {
    if (!workspace) return fail(HGQA_EINVAL, "workspace is NULL");
    if (!aligned16(workspace)) return fail(HGQA_EINVAL, "workspace must be 16-byte aligned");
    if (workspace_bytes < plan.workspace_bytes)
      return fail(HGQA_ENOSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                  plan.workspace_bytes);
  }
  // decode blocks, merge blocks (one per sequence, head and 32 dims), fp32 blocks
  if ((long long)batch * plan.num_splits * l.Hkv > 0x7fffffffLL ||
      (plan.num_splits > 1 && (long long)batch * l.Hq * (l.D / 32) > 0x7fffffffLL) ||
      (long long)batch * l.Hq > 0x7fffffffLL)
    return fail(HGQA_EUNSUPPORTED, "too many decode blocks");
  hgqa::DecodeArgs a{};
  a.q = q;
  a.gate = gate;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.seq_lens = seq_lens;
  a.out = out;
  a.partial = static_cast<float*>(workspace);
  a.B = batch;
  a.Hq = l.Hq;
  a.Hkv = l.Hkv;
  a.G = l.G;
  a.D = l.D;
  a.cap = cache_capacity;
  a.max_seq_len = max_seq_len;
  a.sliding = l.sliding;
  a.window = l.window;
  a.split_keys = plan.split_keys;
  a.num_splits = plan.num_splits;
  a.scale = l.scale;
  fill_rope(l, &a.rope);
  hipError_t e = hgqa::launch_decode(a, l.elem, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(HGQA_EHIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

extern "C" {

const char* hgqa_last_error(void) { return g_last_error.c_str(); }

size_t attn_prefill_workspace_bytes(const hgqa_layer* layer, int32_t batch, int32_t seq_len) {
  Layer l;
  if (check_layer(layer, &l) != HGQA_OK || batch < 0 || seq_len < 0) return 0;
  return prefill_ws(l, batch, seq_len);
}

int attn_prefill(const hgqa_layer* layer, int32_t batch, int32_t seq_len, const void* q,
                 const void* k, const void* v, const void* gate, void* out, void* workspace,
                 size_t workspace_bytes, void* stream) {
  Layer l;
  int rc = check_layer(layer, &l);
  if (rc != HGQA_OK) return rc;
  if (batch < 0 || seq_len < 0) return fail(HGQA_EINVAL, "batch and seq_len must be >= 0");
  if (batch == 0 || seq_len == 0) return ok();
  if (!l.sliding && l.elem == hgqa::Elem::BF16 && l.D == 128 && !uses_vt(l, seq_len))
    return fail(HGQA_EUNSUPPORTED, "a full-layer prompt of %d positions exceeds the V^T limit (2^23)",
                seq_len);
  rc = check_prefill_call(l, batch, seq_len, q, k, v, gate, out, workspace, workspace_bytes,
                          prefill_ws(l, batch, seq_len));
  if (rc != HGQA_OK) return rc;
  hgqa::PrefillArgs a = prefill_args(l, batch, seq_len, q, k, v, gate, out, workspace);
  if (uses_vt(l, seq_len)) {
    a.v_t = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                        rotated_k_bytes(l, batch, seq_len) + table_bytes(l, seq_len));
    a.t_pad = t_pad(seq_len);
  }
  hipError_t e = hgqa::launch_prefill(a, l.elem, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(HGQA_EHIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t attn_prefill_chunk_workspace_bytes(const hgqa_layer* layer, int32_t batch, int32_t n_new,
                                          int32_t max_end_pos) {
  Layer l;
  if (check_layer(layer, &l) != HGQA_OK || batch < 0 || n_new < 0 || max_end_pos < n_new) return 0;
  return chunk_ws(l, batch, n_new) + split_ws(l, batch, n_new, max_end_pos);
}

int attn_prefill_chunk(const hgqa_layer* layer, int32_t batch, int32_t n_new,
                       const int32_t* start_pos, int32_t max_end_pos, const void* q,
                       const void* k, const void* v, const void* gate, void* k_cache,
                       void* v_cache, int32_t cache_capacity, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Layer l;
  int rc = check_layer(layer, &l);
  if (rc != HGQA_OK) return rc;
  if (batch < 0 || n_new < 0) return fail(HGQA_EINVAL, "batch and n_new must be >= 0");
  if (max_end_pos < n_new) return fail(HGQA_EINVAL, "max_end_pos must be >= n_new");
  if (cache_capacity < 1) return fail(HGQA_EINVAL, "cache_capacity must be >= 1");
  if (l.sliding && cache_capacity != l.window)
    return fail(HGQA_EINVAL, "a sliding layer's ring must hold exactly W = %d slots (got %d)",
                l.window, cache_capacity);
  if (!l.sliding && max_end_pos > cache_capacity)
    return fail(HGQA_ENOSPACE, "max_end_pos %d exceeds the full cache capacity %d", max_end_pos,
                cache_capacity);
  if (batch == 0 || n_new == 0) return ok();
  rc = check_prefill_call(l, batch, n_new, q, k, v, gate, out, workspace, workspace_bytes,
                          chunk_ws(l, batch, n_new) + split_ws(l, batch, n_new, max_end_pos));
  if (rc != HGQA_OK) return rc;
  if ((long long)batch * l.Hkv * cache_capacity * l.D > kMaxElems)
    return fail(HGQA_EUNSUPPORTED, "cache too large");
  if (!start_pos) return fail(HGQA_EINVAL, "start_pos is NULL");
  if (!k_cache || !v_cache) return fail(HGQA_EINVAL, "a cache pointer is NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(HGQA_EINVAL, "the caches must be 16-byte aligned");
  const void* caches[2] = {k_cache, v_cache};
  for (const void* c : caches)
    if (c == q || c == k || c == v || c == gate || c == out || c == workspace)
      return fail(HGQA_EINVAL, "a cache must not alias q, k, v, gate, out or the workspace");
  if (k_cache == v_cache) return fail(HGQA_EINVAL, "k_cache and v_cache must differ");

  // A ring still holds the W - 1 positions before the chunk, so there the
  // attention runs first and the chunk joins the cache after it. A full
  // layer's cache has a slot for every position: there the chunk is appended
  // first and the attention reads every key from the cache (bf16, D = 128).
  hgqa::PrefillArgs a = prefill_args(l, batch, n_new, q, k, v, gate, out, workspace);
  if (plan_splits(l, a, max_end_pos) > 0)
    a.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + chunk_ws(l, batch, n_new));
  a.start_pos = start_pos;
  a.max_end_pos = max_end_pos;
  a.cs_bstride = (size_t)n_new * l.half;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cap = cache_capacity;
  a.ring = l.sliding;
  a.keys_in_cache = !l.sliding && l.elem == hgqa::Elem::BF16 && l.D == 128;
  const hipStream_t s = static_cast<hipStream_t>(stream);

  // The chunk joins the cache, as kv_append would leave it.
  hgqa::AppendArgs ap{};
  ap.start_pos = start_pos;
  ap.k_new = k;
  ap.v_new = v;
  ap.k_cache = k_cache;
  ap.v_cache = v_cache;
  ap.B = batch;
  ap.n_new = n_new;
  ap.Hkv = l.Hkv;
  ap.D = l.D;
  ap.cap = cache_capacity;
  ap.sliding = l.sliding;
  ap.window = l.window;
  ap.rope = a.rope;
  hipError_t e;
  if (a.keys_in_cache) {
    e = hgqa::launch_kv_append(ap, l.elem, s);
    if (e != hipSuccess) return fail(HGQA_EHIP, "kv_append launch failed: %s", hipGetErrorString(e));
  }
  e = hgqa::launch_prefill(a, l.elem, s);
  if (e != hipSuccess) return fail(HGQA_EHIP, "prefill launch failed: %s", hipGetErrorString(e));
  if (!a.keys_in_cache) {
    e = hgqa::launch_kv_append(ap, l.elem, s);
    if (e != hipSuccess) return fail(HGQA_EHIP, "kv_append launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

int kv_append(const hgqa_layer* layer, int32_t batch, int32_t n_new, const int32_t* start_pos,
              int32_t max_end_pos, const void* k_new, const void* v_new, void* k_cache,
              void* v_cache, int32_t cache_capacity, void* stream) {
  Layer l;
  int rc = check_layer(layer, &l);
  if (rc != HGQA_OK) return rc;
  if (batch < 0 || n_new < 0) return fail(HGQA_EINVAL, "batch and n_new must be >= 0");
  if (cache_capacity < 1) return fail(HGQA_EINVAL, "cache_capacity must be >= 1");
  if (l.sliding && cache_capacity != l.window)
    return fail(HGQA_EINVAL, "a sliding layer's ring must hold exactly W = %d slots (got %d)",
                l.window, cache_capacity);
  if (max_end_pos < n_new) return fail(HGQA_EINVAL, "max_end_pos must be >= n_new");
  if (!l.sliding && max_end_pos > cache_capacity)
    return fail(HGQA_ENOSPACE, "max_end_pos %d exceeds the full cache capacity %d", max_end_pos,
                cache_capacity);
  if (batch == 0 || n_new == 0) return ok();
  if (batch > 65535) return fail(HGQA_EUNSUPPORTED, "batch %d exceeds 65535", batch);
  if ((long long)batch * l.Hkv * cache_capacity * l.D > kMaxElems)
    return fail(HGQA_EUNSUPPORTED, "cache too large");
  if (!start_pos || !k_new || !v_new || !k_cache || !v_cache)
    return fail(HGQA_EINVAL, "a tensor pointer is NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(HGQA_EINVAL, "k_new, v_new and the caches must be 16-byte aligned");
  hgqa::AppendArgs a{};
  a.start_pos = start_pos;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.B = batch;
  a.n_new = n_new;
  a.Hkv = l.Hkv;
  a.D = l.D;
  a.cap = cache_capacity;
  a.sliding = l.sliding;
  a.window = l.window;
  fill_rope(l, &a.rope);
  hipError_t e = hgqa::launch_kv_append(a, l.elem, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(HGQA_EHIP, "kv_append launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t attn_decode_workspace_bytes(const hgqa_layer* layer, int32_t batch, int32_t max_seq_len) {
  Layer l;
  if (check_layer(layer, &l) != HGQA_OK || batch < 1 || max_seq_len < 1) return 0;
  return hgqa::plan_decode(l.elem, batch, l.Hq, l.Hkv, l.D, l.sliding, l.window, max_seq_len,
                           g_decode_split_keys.load(std::memory_order_relaxed))
      .workspace_bytes;
}

int attn_decode(const hgqa_layer* layer, int32_t batch, const void* q, const void* gate,
                const void* k_cache, const void* v_cache, int32_t cache_capacity,
                const int32_t* seq_lens, int32_t max_seq_len, void* workspace,
                size_t workspace_bytes, void* out, void* stream) {
  return hgqa::decode_call(layer, batch, q, gate, k_cache, v_cache, cache_capacity, seq_lens,
                           max_seq_len, workspace, workspace_bytes, out, stream, nullptr, 0);
}

int hgqa_set_tuning(int32_t knob, int32_t value) {
  switch (knob) {
    case HGQA_TUNE_PREFILL_WAVES:
      if (value != 0 && value != 4 && value != 8)
        return fail(HGQA_EINVAL, "HGQA_TUNE_PREFILL_WAVES takes 0, 4 or 8 (got %d)", value);
      g_prefill_waves.store(value, std::memory_order_relaxed);
      return ok();
    case HGQA_TUNE_DECODE_SPLIT_KEYS:
      if (value < 0) return fail(HGQA_EINVAL, "HGQA_TUNE_DECODE_SPLIT_KEYS must be >= 0");
      g_decode_split_keys.store(value, std::memory_order_relaxed);
      return ok();
    case HGQA_TUNE_CHUNK_SPLIT_TILES:
      if (value < 0) return fail(HGQA_EINVAL, "HGQA_TUNE_CHUNK_SPLIT_TILES must be >= 0");
      g_chunk_split_tiles.store(value, std::memory_order_relaxed);
      return ok();
    default:
      return fail(HGQA_EINVAL, "unknown tuning knob %d", knob);
  }
}

}  // extern "C"
