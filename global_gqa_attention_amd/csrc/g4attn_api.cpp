// g4attn_api.cpp -- the C ABI: host-side validation, provenance and launches.
//
// Every check runs before any HIP call, so a rejected request launches nothing and
// touches no output (RL-Kernel issue #415, section 4, rule 7: unsupported strict geometry
// fails closed). Provenance (rule 8) reports the implementation, tile shape, split
// policy and accumulator type of each launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/g4attn.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

g4attn_status fail(g4attn_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

g4attn_status ok() {
  g_last_error.clear();
  return G4ATTN_OK;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Geometry shared by every entry point.
g4attn_status check_layer(const g4attn_layer* L) {
  if (!L) return fail(G4ATTN_ERR_INVALID_ARG, "layer descriptor is NULL");
  if (L->kind != G4ATTN_SLIDING && L->kind != G4ATTN_GLOBAL)
    return fail(G4ATTN_ERR_INVALID_ARG, "layer kind %d is neither sliding (0) nor global (1)", L->kind);
  if (L->v_norm != 0 && L->v_norm != 1) return fail(G4ATTN_ERR_INVALID_ARG, "v_norm must be 0 or 1");
  if (L->num_q_heads <= 0 || L->num_kv_heads <= 0)
    return fail(G4ATTN_ERR_INVALID_ARG, "head counts must be positive (q %d, kv %d)", L->num_q_heads,
                L->num_kv_heads);
  if (L->num_q_heads % L->num_kv_heads != 0)
    return fail(G4ATTN_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", L->num_q_heads,
                L->num_kv_heads);
  const int G = L->num_q_heads / L->num_kv_heads;
  if (!is_pow2(G) || G > 32)
    return fail(G4ATTN_ERR_UNSUPPORTED, "query heads per KV head %d: supported are 1, 2, 4, 8, 16, 32", G);
  const int D = L->head_dim;
  if (D != 64 && D != 128 && D != 256 && D != 512)
    return fail(G4ATTN_ERR_UNSUPPORTED, "head_dim %d: supported are 64, 128, 256, 512", D);
  if (L->window < 0) return fail(G4ATTN_ERR_INVALID_ARG, "window %d is negative", L->window);
  if (L->kind == G4ATTN_SLIDING && L->window == 0)
    return fail(G4ATTN_ERR_INVALID_ARG, "a sliding layer needs window > 0");
  if (L->kind == G4ATTN_GLOBAL && L->window != 0)
    return fail(G4ATTN_ERR_INVALID_ARG, "a global layer has window 0 (full causal), got %d", L->window);
  if (L->k_eq_v != 0 && L->k_eq_v != 1) return fail(G4ATTN_ERR_INVALID_ARG, "k_eq_v must be 0 or 1");
  if (L->k_eq_v && L->v_norm) return fail(G4ATTN_ERR_INVALID_ARG, "v_norm needs a separate V (k_eq_v == 0)");
  if (!(std::isfinite(L->softmax_scale) && L->softmax_scale > 0.0f))
    return fail(G4ATTN_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (!(std::isfinite(L->rms_eps) && L->rms_eps >= 0.0f))
    return fail(G4ATTN_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  const int R = L->rope_dims;
  if (R < 0 || R > D || (R & 1)) return fail(G4ATTN_ERR_INVALID_ARG, "rope_dims %d must be even and in [0, %d]", R, D);
  if (R > 0) {
    if (L->rope_freq_dim <= 0) return fail(G4ATTN_ERR_INVALID_ARG, "rope_freq_dim must be > 0");
    if (!(std::isfinite(L->rope_theta) && L->rope_theta > 0.0))
      return fail(G4ATTN_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
    if (L->rope_pairing != G4ATTN_ROPE_PAIRS_IN_BLOCK && L->rope_pairing != G4ATTN_ROPE_PAIRS_HALF_HEAD)
      return fail(G4ATTN_ERR_INVALID_ARG, "rope_pairing %d unknown", L->rope_pairing);
    // The prologue gives each lane 8 consecutive dims of a row: a lane's dims must all
    // rotate or all not, and its partner sits a power-of-two number of lanes away.
    const int per_lane = 8;
    const int P = L->rope_pairing == G4ATTN_ROPE_PAIRS_HALF_HEAD ? D / 2 : R / 2;
    if ((R / 2) % per_lane != 0 || P % per_lane != 0 || !is_pow2(P / per_lane))
      return fail(G4ATTN_ERR_UNSUPPORTED, "rope_dims %d with head_dim %d: R/2 must be a multiple of 8 and the "
                  "pair offset a power-of-two multiple of 8", R, D);
  }
  return G4ATTN_OK;
}

int pair_offset(const g4attn_layer* L) {
  return L->rope_pairing == G4ATTN_ROPE_PAIRS_HALF_HEAD ? L->head_dim / 2 : L->rope_dims / 2;
}

uint64_t fnv1a(uint64_t h, const void* p, size_t n) {
  const unsigned char* c = static_cast<const unsigned char*>(p);
  for (size_t i = 0; i < n; ++i) {
    h ^= c[i];
    h *= 1099511628211ull;
  }
  return h;
}

void fill_provenance(g4attn_provenance* prov, const g4attn_layer* L, const g4::LaunchShape& shape,
                     int64_t extent, int32_t split_keys = 0) {
  if (!prov) return;
  std::memset(prov, 0, sizeof *prov);
  std::snprintf(prov->kernel_id, sizeof prov->kernel_id, "g4attn.%s", shape.kernel_name);
  prov->kind = L->kind;
  prov->head_dim = L->head_dim;
  prov->group = L->num_q_heads / L->num_kv_heads;
  prov->block_q = shape.block_q;
  prov->block_k = shape.block_k;
  prov->mfma_m = 32;
  prov->mfma_n = 32;
  prov->mfma_k = 16;
  prov->waves_per_group = shape.waves;
  prov->split_kv = split_keys;
  prov->acc_fp32 = 1;
  prov->fallback = 0;
  uint64_t h = 1469598103934665603ull;
  h = fnv1a(h, L, sizeof *L);
  h = fnv1a(h, &extent, sizeof extent);
  h = fnv1a(h, &split_keys, sizeof split_keys);
  prov->shape_fingerprint = h;
}

constexpr double kLog2e = 1.4426950408889634;
constexpr uint64_t kMaxBufferBytes = 0x7FFFFFFFull;  // buffer offsets are 32-bit

// Compute units of each device, read once per device (0: not read yet).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Whether a prefill grid of `groups` work-groups (two N-blocks per wave) leaves CUs of
// the current device without one: then the narrow form, one N-block per wave and twice
// the work-groups, is launched. Rows get the same bits from either form.
bool narrow_grid(int head_dim, int64_t groups) {
  if (head_dim >= 512) return false;  // the 512-dim head always takes one N-block per wave
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  return groups < cu_count(dev);
}

// The prefill entry points write `out` while other work-groups still read k and v (and
// their own q rows): the output must be a buffer of its own. Only identical base
// pointers can be seen on the host (the row counts live on the device); partial overlaps
// are the caller's to avoid.
g4attn_status check_out_alias(const void* out, const void* q, const void* k, const void* v) {
  if (out == q || out == k || (v && out == v))
    return fail(G4ATTN_ERR_INVALID_ARG, "out must not be q, k or v (prefill is not in place)");
  return G4ATTN_OK;
}

// The split form's request: chunk size and the caller's workspace.
struct SplitRequest {
  int32_t keys;
  void* workspace;
  uint64_t workspace_bytes;
};

// Partial layout of a split call: `rows` row slots per sequence, one chunk slot per
// chunk of the longest key range; bytes = partials x (D + 2) x 4 (0: no row has keys in
// two chunks, nothing is split).
struct SplitLayout {
  int64_t chunks;
  int64_t partials;
  uint64_t bytes;
};

SplitLayout split_layout(const g4attn_layer* layer, int64_t batch, int64_t rows, int64_t max_key_len, int32_t keys) {
  SplitLayout s{};
  s.chunks = max_key_len > 0 ? (max_key_len + keys - 1) / keys : 0;
  if (s.chunks < 2 || batch == 0 || rows == 0) return SplitLayout{s.chunks, 0, 0};
  s.partials = batch * rows * layer->num_q_heads * s.chunks;
  s.bytes = (uint64_t)s.partials * (uint64_t)(layer->head_dim + 2) * 4u;
  return s;
}

g4attn_status check_split(const g4attn_layer* layer, int32_t keys) {
  if (keys <= 0 || keys % 256 != 0)
    return fail(G4ATTN_ERR_INVALID_ARG, "split_keys %d must be a positive multiple of 256", keys);
  if (layer->window != 0)
    return fail(G4ATTN_ERR_UNSUPPORTED, "the split form is for global layers (window 0), got window %d",
                layer->window);
  return G4ATTN_OK;
}

// The workspace of a split call that splits: present, large enough, not an input or output.
g4attn_status check_workspace(const SplitRequest& sp, const SplitLayout& lay, const void* a, const void* b,
                              const void* c, const void* d) {
  if (lay.bytes == 0) return G4ATTN_OK;
  if (!sp.workspace) return fail(G4ATTN_ERR_INVALID_ARG, "workspace is NULL (%llu bytes needed)",
                                 (unsigned long long)lay.bytes);
  if (sp.workspace_bytes < lay.bytes)
    return fail(G4ATTN_ERR_INVALID_ARG, "workspace of %llu bytes, %llu needed", (unsigned long long)sp.workspace_bytes,
                (unsigned long long)lay.bytes);
  if (reinterpret_cast<uintptr_t>(sp.workspace) % 16 != 0)
    return fail(G4ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (sp.workspace == a || sp.workspace == b || (c && sp.workspace == c) || (d && sp.workspace == d))
    return fail(G4ATTN_ERR_INVALID_ARG, "workspace must not be an input or output of the call");
  return G4ATTN_OK;
}

g4::SplitArgs split_args(const g4attn_layer* layer, const SplitRequest& sp, const SplitLayout& lay, int32_t rows) {
  g4::SplitArgs s{};
  s.keys = sp.keys;
  s.chunks = (int32_t)lay.chunks;
  s.rows = rows;
  s.part_o = static_cast<float*>(sp.workspace);
  s.part_ml = s.part_o + lay.partials * layer->head_dim;
  return s;
}

// Packed varlen prefill with optional per-row last keys (null: causal rows).
// With `sp` (the split form): chunk work-groups and the merge when some row's keys span
// two chunks, else the plain kernels (every row then has one chunk: the same bits).
// The q prologue inside the prefill (g4attn_prefill_qp).
struct QpRequest {
  const uint16_t* q_norm_w;
  const int32_t* positions;
};

g4attn_status prefill_impl(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           uint16_t* out, const int32_t* seq_start, const int32_t* seq_len, const int32_t* last_key,
                           int32_t batch, int32_t max_seq_len, g4attn_stream_t stream, g4attn_provenance* prov,
                           const SplitRequest* sp = nullptr, const QpRequest* qp = nullptr) {
  if (g4attn_status s = check_layer(layer)) return s;
  if (qp) {
    if (layer->head_dim != 512 || !layer->k_eq_v)
      return fail(G4ATTN_ERR_UNSUPPORTED, "the q prologue inside the prefill needs head dim 512 with K=V");
    // the angle tables (cos and sin, fp32, per position of a work-group's rows and rotated
    // pair) and q_norm_w share the first 32 KiB key stage
    const int64_t ppg = g4::prefill_rows_per_group(512, true, false) / (layer->num_q_heads / layer->num_kv_heads);
    if (4 * ppg * (layer->rope_dims / 2) + 4 * ((ppg * (layer->rope_dims / 2) + 3) & ~3) + 2 * 512 > 32768)
      return fail(G4ATTN_ERR_UNSUPPORTED, "the q prologue inside the prefill: rope_dims %d too large for group size %d",
                  layer->rope_dims, layer->num_q_heads / layer->num_kv_heads);
    if (batch > 0 && (!qp->q_norm_w || !qp->positions))
      return fail(G4ATTN_ERR_INVALID_ARG, "q_norm_w / positions are NULL");
  }
  if (sp) {
    if (g4attn_status s = check_split(layer, sp->keys)) return s;
  }
  if (batch < 0) return fail(G4ATTN_ERR_INVALID_ARG, "batch %d is negative", batch);
  if (max_seq_len < 0) return fail(G4ATTN_ERR_INVALID_ARG, "max_seq_len %d is negative", max_seq_len);
  if (!q || !k || !out) return fail(G4ATTN_ERR_INVALID_ARG, "q, k and out must not be NULL");
  if (layer->k_eq_v && v) return fail(G4ATTN_ERR_INVALID_ARG, "v must be NULL for a K=V layer");
  if (!layer->k_eq_v && !v) return fail(G4ATTN_ERR_INVALID_ARG, "v is NULL for a layer with separate K and V");
  if (batch > 0 && (!seq_start || !seq_len)) return fail(G4ATTN_ERR_INVALID_ARG, "seq_start / seq_len are NULL");
  const int D = layer->head_dim;
  // (No bound on the sequence's K/V span: every buffer descriptor of the kernels covers
  // one 32-key block or one work-group's query rows, placed by a 64-bit pointer shift.)
  const int G = layer->num_q_heads / layer->num_kv_heads;
  const int rows = g4::prefill_rows_per_group(D, layer->k_eq_v != 0, false);
  int64_t qblocks = ((int64_t)max_seq_len * G + rows - 1) / rows;
  const int64_t groups = qblocks * batch * layer->num_kv_heads;
  if (groups > 0x7FFFFFFF) return fail(G4ATTN_ERR_UNSUPPORTED, "grid too large");
  const int32_t split_keys = sp ? sp->keys : 0;
  const SplitLayout lay = sp ? split_layout(layer, batch, max_seq_len, max_seq_len, sp->keys) : SplitLayout{};
  if (lay.bytes > 0 && groups * lay.chunks > 0x7FFFFFFF) return fail(G4ATTN_ERR_UNSUPPORTED, "grid too large");
  g4::LaunchShape shape{};
  if (batch == 0 || max_seq_len == 0) {
    if (prov) {
      shape.kernel_name = "prefill.empty";
      fill_provenance(prov, layer, shape, 0, split_keys);
    }
    return ok();
  }
  if (g4attn_status s = check_out_alias(out, q, k, v)) return s;
  if (sp) {
    if (g4attn_status s = check_workspace(*sp, lay, q, k, v, out)) return s;
  }
  g4::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = layer->k_eq_v ? k : v;
  a.out = out;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.q_pos0 = nullptr;
  a.kv_row0 = nullptr;
  a.kv_slots = 0;
  a.last_key = last_key;
  a.num_q_heads = layer->num_q_heads;
  a.num_kv_heads = layer->num_kv_heads;
  a.window = layer->window;
  a.num_qblocks = (int32_t)qblocks;
  a.batch = batch;
  a.scale_log2 = (float)((double)layer->softmax_scale * kLog2e);
  if (lay.bytes > 0) {
    a.split = split_args(layer, *sp, lay, max_seq_len);
    g4::MergeArgs m{};
    m.part_o = a.split.part_o;
    m.part_ml = a.split.part_ml;
    m.out = out;
    m.out_row0 = seq_start;
    m.nrows = seq_len;
    m.pos_ref = nullptr;
    m.pos_bias = 0;
    m.num_q_heads = layer->num_q_heads;
    m.batch = batch;
    m.rows = max_seq_len;
    m.chunks = a.split.chunks;
    m.split_keys = sp->keys;
    m.row_skip = std::min(sp->keys, max_seq_len);  // (row i sits at position i)
    const hipError_t e =
        g4::launch_prefill_split(D, layer->k_eq_v != 0, a, m, reinterpret_cast<hipStream_t>(stream), &shape);
    if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
    fill_provenance(prov, layer, shape, (int64_t)max_seq_len * batch, split_keys);
    return ok();
  }
  if (qp) {
    // (head dim 512: one N-block per wave already, no narrow form)
    a.q_norm_w = qp->q_norm_w;
    a.positions = qp->positions;
    a.rope_dims = layer->rope_dims;
    a.rope_freq_dim = layer->rope_freq_dim > 0 ? layer->rope_freq_dim : 1;
    a.pair_offset = layer->rope_dims > 0 ? pair_offset(layer) : 0;
    a.rope_theta = layer->rope_theta;
    a.rms_eps = layer->rms_eps;
    const hipError_t e = g4::launch_prefill_qp(a, reinterpret_cast<hipStream_t>(stream), &shape);
    if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
    fill_provenance(prov, layer, shape, (int64_t)max_seq_len * batch, split_keys);
    return ok();
  }
  const bool narrow = narrow_grid(D, groups);
  if (narrow) {
    const int nrows = g4::prefill_rows_per_group(D, layer->k_eq_v != 0, true);
    qblocks = ((int64_t)a.num_qblocks * rows + nrows - 1) / nrows;
    a.num_qblocks = (int32_t)qblocks;
  }
  const hipError_t e =
      g4::launch_prefill(D, layer->k_eq_v != 0, narrow, a, reinterpret_cast<hipStream_t>(stream), &shape);
  if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
  fill_provenance(prov, layer, shape, (int64_t)max_seq_len * batch, split_keys);
  return ok();
}


// Chunked prefill against the cache, with optional per-row last keys (null: causal rows).
g4attn_status cached_impl(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                          const uint16_t* v_cache, uint16_t* out, const int32_t* q_row0, const int32_t* q_pos0,
                          const int32_t* chunk_len, const int32_t* last_key, const int64_t* cache_row0,
                          int32_t cache_slots, int32_t batch, int32_t max_chunk_len, int32_t max_key_len,
                          g4attn_stream_t stream, g4attn_provenance* prov, const SplitRequest* sp = nullptr) {
  if (g4attn_status s = check_layer(layer)) return s;
  if (sp) {
    if (g4attn_status s = check_split(layer, sp->keys)) return s;
  }
  if (batch < 0) return fail(G4ATTN_ERR_INVALID_ARG, "batch %d is negative", batch);
  if (max_chunk_len < 0) return fail(G4ATTN_ERR_INVALID_ARG, "max_chunk_len %d is negative", max_chunk_len);
  if (max_key_len < max_chunk_len)
    return fail(G4ATTN_ERR_INVALID_ARG, "max_key_len %d is below max_chunk_len %d", max_key_len, max_chunk_len);
  if (!q || !k_cache || !out) return fail(G4ATTN_ERR_INVALID_ARG, "q, k_cache and out must not be NULL");
  if (layer->k_eq_v && v_cache) return fail(G4ATTN_ERR_INVALID_ARG, "v_cache must be NULL for a K=V layer");
  if (!layer->k_eq_v && !v_cache) return fail(G4ATTN_ERR_INVALID_ARG, "v_cache is NULL for separate K and V");
  if (batch > 0 && (!q_row0 || !q_pos0 || !chunk_len || !cache_row0))
    return fail(G4ATTN_ERR_INVALID_ARG, "q_row0 / q_pos0 / chunk_len / cache_row0 are NULL");
  if (cache_slots <= 0 || cache_slots % 32 != 0)
    return fail(G4ATTN_ERR_INVALID_ARG, "cache_slots %d must be a positive multiple of 32", cache_slots);
  if (layer->window > 0 && (int64_t)cache_slots < (int64_t)layer->window + max_chunk_len)
    return fail(G4ATTN_ERR_INVALID_ARG, "a ring of %d slots cannot hold a window of %d plus a chunk of %d",
                cache_slots, layer->window, max_chunk_len);
  if (layer->window == 0 && cache_slots < max_key_len)
    return fail(G4ATTN_ERR_INVALID_ARG, "a linear cache of %d slots cannot hold %d positions", cache_slots,
                max_key_len);
  const int D = layer->head_dim;
  const int G = layer->num_q_heads / layer->num_kv_heads;
  const int rows = g4::prefill_rows_per_group(D, layer->k_eq_v != 0, false);
  int64_t qblocks = ((int64_t)max_chunk_len * G + rows - 1) / rows;
  const int64_t groups = qblocks * batch * layer->num_kv_heads;
  if (groups > 0x7FFFFFFF) return fail(G4ATTN_ERR_UNSUPPORTED, "grid too large");
  const int32_t split_keys = sp ? sp->keys : 0;
  const SplitLayout lay = sp ? split_layout(layer, batch, max_chunk_len, max_key_len, sp->keys) : SplitLayout{};
  if (lay.bytes > 0 && groups * lay.chunks > 0x7FFFFFFF) return fail(G4ATTN_ERR_UNSUPPORTED, "grid too large");
  g4::LaunchShape shape{};
  if (batch == 0 || max_chunk_len == 0) {
    if (prov) {
      shape.kernel_name = "prefill.empty";
      fill_provenance(prov, layer, shape, 0, split_keys);
    }
    return ok();
  }
  if (g4attn_status s = check_out_alias(out, q, k_cache, v_cache)) return s;
  if (sp) {
    if (g4attn_status s = check_workspace(*sp, lay, q, k_cache, v_cache, out)) return s;
  }
  g4::PrefillArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = layer->k_eq_v ? k_cache : v_cache;
  a.out = out;
  a.seq_start = q_row0;
  a.seq_len = chunk_len;
  a.q_pos0 = q_pos0;
  a.kv_row0 = cache_row0;
  a.kv_slots = cache_slots;
  a.last_key = last_key;
  a.num_q_heads = layer->num_q_heads;
  a.num_kv_heads = layer->num_kv_heads;
  a.window = layer->window;
  a.num_qblocks = (int32_t)qblocks;
  a.batch = batch;
  a.scale_log2 = (float)((double)layer->softmax_scale * kLog2e);
  if (lay.bytes > 0) {
    a.split = split_args(layer, *sp, lay, max_chunk_len);
    g4::MergeArgs m{};
    m.part_o = a.split.part_o;
    m.part_ml = a.split.part_ml;
    m.out = out;
    m.out_row0 = q_row0;
    m.nrows = chunk_len;
    m.pos_ref = q_pos0;
    m.pos_bias = 0;
    m.num_q_heads = layer->num_q_heads;
    m.batch = batch;
    m.rows = max_chunk_len;
    m.chunks = a.split.chunks;
    m.split_keys = sp->keys;
    const hipError_t e =
        g4::launch_prefill_split(D, layer->k_eq_v != 0, a, m, reinterpret_cast<hipStream_t>(stream), &shape);
    if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
    fill_provenance(prov, layer, shape, (int64_t)max_chunk_len * batch, split_keys);
    return ok();
  }
  const bool narrow = narrow_grid(D, groups);
  if (narrow) {
    const int nrows = g4::prefill_rows_per_group(D, layer->k_eq_v != 0, true);
    qblocks = ((int64_t)a.num_qblocks * rows + nrows - 1) / nrows;
    a.num_qblocks = (int32_t)qblocks;
  }
  const hipError_t e =
      g4::launch_prefill(D, layer->k_eq_v != 0, narrow, a, reinterpret_cast<hipStream_t>(stream), &shape);
  if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
  fill_provenance(prov, layer, shape, (int64_t)max_chunk_len * batch, split_keys);
  return ok();
}

// One new token per sequence; with `sp` the split form (chunk work-groups and the merge
// when some sequence's keys span two chunks).
g4attn_status decode_impl(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                          const uint16_t* v_cache, const int64_t* cache_row0, const int32_t* ctx_len,
                          int32_t cache_slots, uint16_t* out, int32_t batch, int32_t max_ctx_len,
                          const int32_t* schedule, g4attn_stream_t stream, g4attn_provenance* prov,
                          const SplitRequest* sp) {
  if (g4attn_status s = check_layer(layer)) return s;
  if (sp) {
    if (g4attn_status s = check_split(layer, sp->keys)) return s;
  }
  if (batch < 0) return fail(G4ATTN_ERR_INVALID_ARG, "batch %d is negative", batch);
  if (!q || !k_cache || !out) return fail(G4ATTN_ERR_INVALID_ARG, "q, k_cache and out must not be NULL");
  if (layer->k_eq_v && v_cache) return fail(G4ATTN_ERR_INVALID_ARG, "v_cache must be NULL for a K=V layer");
  if (!layer->k_eq_v && !v_cache) return fail(G4ATTN_ERR_INVALID_ARG, "v_cache is NULL for separate K and V");
  if (batch > 0 && (!cache_row0 || !ctx_len)) return fail(G4ATTN_ERR_INVALID_ARG, "cache_row0 / ctx_len are NULL");
  if (cache_slots <= 0) return fail(G4ATTN_ERR_INVALID_ARG, "cache_slots %d must be > 0", cache_slots);
  if (batch > 0 && max_ctx_len <= 0) return fail(G4ATTN_ERR_INVALID_ARG, "max_ctx_len must be >= 1");
  if (layer->window > 0 && cache_slots < layer->window)
    return fail(G4ATTN_ERR_INVALID_ARG, "a ring of %d slots cannot hold a window of %d", cache_slots, layer->window);
  if (layer->window == 0 && cache_slots < max_ctx_len)
    return fail(G4ATTN_ERR_INVALID_ARG, "a linear cache of %d slots cannot hold %d positions", cache_slots,
                max_ctx_len);
  const int D = layer->head_dim;
  const uint64_t stride = (uint64_t)layer->num_kv_heads * D * 2;
  if ((uint64_t)cache_slots * stride > kMaxBufferBytes)
    return fail(G4ATTN_ERR_UNSUPPORTED, "a sequence's cache span exceeds 2 GiB (32-bit buffer offsets)");
  const int64_t groups = (int64_t)batch * layer->num_kv_heads;
  if (groups > 0x7FFFFFFF) return fail(G4ATTN_ERR_UNSUPPORTED, "grid too large");
  const int32_t split_keys = sp ? sp->keys : 0;
  const SplitLayout lay = sp ? split_layout(layer, batch, 1, max_ctx_len, sp->keys) : SplitLayout{};
  if (lay.bytes > 0 && groups * lay.chunks > 0x7FFFFFFF) return fail(G4ATTN_ERR_UNSUPPORTED, "grid too large");
  g4::LaunchShape shape{};
  if (batch == 0) {
    if (prov) {
      shape.kernel_name = "decode.empty";
      fill_provenance(prov, layer, shape, 0, split_keys);
    }
    return ok();
  }
  if (sp) {
    if (out == q || out == k_cache || (v_cache && out == v_cache))
      return fail(G4ATTN_ERR_INVALID_ARG, "out must not be q or a cache in the split form");
    if (g4attn_status s = check_workspace(*sp, lay, q, k_cache, v_cache, out)) return s;
  }
  g4::DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = layer->k_eq_v ? k_cache : v_cache;
  a.out = out;
  a.cache_row0 = cache_row0;
  a.ctx_len = ctx_len;
  a.schedule = schedule;
  a.num_q_heads = layer->num_q_heads;
  a.num_kv_heads = layer->num_kv_heads;
  a.window = layer->window;
  a.cache_slots = cache_slots;
  a.batch = batch;
  a.scale_log2 = (float)((double)layer->softmax_scale * kLog2e);
  if (lay.bytes > 0) {
    a.split = split_args(layer, *sp, lay, 1);
    g4::MergeArgs m{};
    m.part_o = a.split.part_o;
    m.part_ml = a.split.part_ml;
    m.out = out;
    m.out_row0 = nullptr;
    m.nrows = nullptr;
    m.pos_ref = ctx_len;
    m.pos_bias = -1;
    m.num_q_heads = layer->num_q_heads;
    m.batch = batch;
    m.rows = 1;
    m.chunks = a.split.chunks;
    m.split_keys = sp->keys;
    const hipError_t e =
        g4::launch_decode_split(D, layer->k_eq_v != 0, a, m, reinterpret_cast<hipStream_t>(stream), &shape);
    if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "decode launch failed: %s", hipGetErrorString(e));
    fill_provenance(prov, layer, shape, (int64_t)max_ctx_len * batch, split_keys);
    return ok();
  }
  const hipError_t e = g4::launch_decode(D, layer->k_eq_v != 0, a, reinterpret_cast<hipStream_t>(stream), &shape);
  if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "decode launch failed: %s", hipGetErrorString(e));
  fill_provenance(prov, layer, shape, (int64_t)max_ctx_len * batch, split_keys);
  return ok();
}

}  // namespace

extern "C" {

int32_t g4attn_abi_version(void) { return G4ATTN_ABI_VERSION; }

const char* g4attn_last_error(void) { return g_last_error.c_str(); }

g4attn_status g4attn_qk_prologue(const g4attn_layer* layer, const uint16_t* q_in, uint16_t* q_out,
                                 const uint16_t* k_in, uint16_t* k_out, const uint16_t* v_in, uint16_t* v_out,
                                 const uint16_t* q_norm_w, const uint16_t* k_norm_w, const int32_t* positions,
                                 const int64_t* kv_dst_row, int64_t num_tokens, g4attn_stream_t stream) {
  if (g4attn_status s = check_layer(layer)) return s;
  if (num_tokens < 0) return fail(G4ATTN_ERR_INVALID_ARG, "num_tokens %lld is negative", (long long)num_tokens);
  if (num_tokens > 0x7FFFFFFF) return fail(G4ATTN_ERR_UNSUPPORTED, "num_tokens above 2^31 - 1");
  if ((q_in == nullptr) != (q_out == nullptr)) return fail(G4ATTN_ERR_INVALID_ARG, "q_in and q_out: both or neither");
  if ((k_in == nullptr) != (k_out == nullptr)) return fail(G4ATTN_ERR_INVALID_ARG, "k_in and k_out: both or neither");
  if ((v_in == nullptr) != (v_out == nullptr)) return fail(G4ATTN_ERR_INVALID_ARG, "v_in and v_out: both or neither");
  if (!q_in && !k_in && !v_in) return fail(G4ATTN_ERR_INVALID_ARG, "nothing to do: q, k and v are all NULL");
  if (q_in && !q_norm_w) return fail(G4ATTN_ERR_INVALID_ARG, "q_norm_w is NULL");
  if (k_in && !k_norm_w) return fail(G4ATTN_ERR_INVALID_ARG, "k_norm_w is NULL");
  if (v_in && layer->k_eq_v) return fail(G4ATTN_ERR_INVALID_ARG, "v given for a K=V layer");
  if (!positions) return fail(G4ATTN_ERR_INVALID_ARG, "positions is NULL");
  if (kv_dst_row && (k_in == k_out || (v_in && v_in == v_out)))
    return fail(G4ATTN_ERR_INVALID_ARG, "a scattered k/v write (kv_dst_row) cannot be in place");
  if (num_tokens == 0) return ok();
  g4::PrologueArgs a{};
  a.q_in = q_in;
  a.q_out = q_out;
  a.k_in = k_in;
  a.k_out = k_out;
  a.v_in = v_in;
  a.v_out = v_out;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.positions = positions;
  a.kv_dst_row = kv_dst_row;
  a.num_tokens = num_tokens;
  a.num_q_heads = layer->num_q_heads;
  a.num_kv_heads = layer->num_kv_heads;
  a.rope_dims = layer->rope_dims;
  a.rope_freq_dim = layer->rope_freq_dim > 0 ? layer->rope_freq_dim : 1;
  a.pair_offset = layer->rope_dims > 0 ? pair_offset(layer) : 0;
  a.rope_theta = layer->rope_theta;
  a.rms_eps = layer->rms_eps;
  a.v_norm = layer->v_norm;
  const hipError_t e = g4::launch_prologue(layer->head_dim, a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "prologue launch failed: %s", hipGetErrorString(e));
  return ok();
}


g4attn_status g4attn_prefill(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, const int32_t* seq_start, const int32_t* seq_len, int32_t batch,
                             int32_t max_seq_len, g4attn_stream_t stream, g4attn_provenance* prov) {
  return prefill_impl(layer, q, k, v, out, seq_start, seq_len, nullptr, batch, max_seq_len, stream, prov);
}

g4attn_status g4attn_prefill_qp(const g4attn_layer* layer, const uint16_t* q, const uint16_t* q_norm_w,
                                const int32_t* positions, const uint16_t* k, const uint16_t* v, uint16_t* out,
                                const int32_t* seq_start, const int32_t* seq_len, int32_t batch,
                                int32_t max_seq_len, g4attn_stream_t stream, g4attn_provenance* prov) {
  const QpRequest qp{q_norm_w, positions};
  return prefill_impl(layer, q, k, v, out, seq_start, seq_len, nullptr, batch, max_seq_len, stream, prov, nullptr, &qp);
}

g4attn_status g4attn_prefill_masked(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k,
                                    const uint16_t* v, uint16_t* out, const int32_t* seq_start,
                                    const int32_t* seq_len, const int32_t* last_key, int32_t batch,
                                    int32_t max_seq_len, g4attn_stream_t stream, g4attn_provenance* prov) {
  if (batch > 0 && !last_key) return fail(G4ATTN_ERR_INVALID_ARG, "last_key is NULL");
  return prefill_impl(layer, q, k, v, out, seq_start, seq_len, last_key, batch, max_seq_len, stream, prov);
}


g4attn_status g4attn_prefill_cached(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                    const uint16_t* v_cache, uint16_t* out, const int32_t* q_row0,
                                    const int32_t* q_pos0, const int32_t* chunk_len, const int64_t* cache_row0,
                                    int32_t cache_slots, int32_t batch, int32_t max_chunk_len, int32_t max_key_len,
                                    g4attn_stream_t stream, g4attn_provenance* prov) {
  return cached_impl(layer, q, k_cache, v_cache, out, q_row0, q_pos0, chunk_len, nullptr, cache_row0, cache_slots,
                     batch, max_chunk_len, max_key_len, stream, prov);
}

g4attn_status g4attn_prefill_cached_masked(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                           const uint16_t* v_cache, uint16_t* out, const int32_t* q_row0,
                                           const int32_t* q_pos0, const int32_t* chunk_len, const int32_t* last_key,
                                           const int64_t* cache_row0, int32_t cache_slots, int32_t batch,
                                           int32_t max_chunk_len, int32_t max_key_len, g4attn_stream_t stream,
                                           g4attn_provenance* prov) {
  if (batch > 0 && !last_key) return fail(G4ATTN_ERR_INVALID_ARG, "last_key is NULL");
  return cached_impl(layer, q, k_cache, v_cache, out, q_row0, q_pos0, chunk_len, last_key, cache_row0,
                     cache_slots, batch, max_chunk_len, max_key_len, stream, prov);
}

g4attn_status g4attn_prefill_backward(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const uint16_t* out, const uint16_t* dout, uint16_t* dq,
                                      uint16_t* dk, uint16_t* dv, float* lse, float* delta, const int32_t* seq_start,
                                      const int32_t* seq_len, int32_t batch, int32_t max_seq_len,
                                      g4attn_stream_t stream) {
  if (g4attn_status s = check_layer(layer)) return s;
  if (batch < 0) return fail(G4ATTN_ERR_INVALID_ARG, "batch %d is negative", batch);
  if (max_seq_len < 0) return fail(G4ATTN_ERR_INVALID_ARG, "max_seq_len %d is negative", max_seq_len);
  if (!q || !k || !out || !dout || !dq || !dk || !lse || !delta)
    return fail(G4ATTN_ERR_INVALID_ARG, "q, k, out, dout, dq, dk, lse and delta must not be NULL");
  if (layer->k_eq_v && (v || dv)) return fail(G4ATTN_ERR_INVALID_ARG, "v and dv must be NULL for a K=V layer");
  if (!layer->k_eq_v && (!v || !dv))
    return fail(G4ATTN_ERR_INVALID_ARG, "v and dv are needed for a layer with separate K and V");
  if (batch > 0 && (!seq_start || !seq_len)) return fail(G4ATTN_ERR_INVALID_ARG, "seq_start / seq_len are NULL");
  const void* ins[] = {q, k, v, out, dout};
  const void* outs[] = {dq, dk, dv, lse, delta};
  for (const void* o : outs) {
    if (!o) continue;
    for (const void* i : ins)
      if (o == i) return fail(G4ATTN_ERR_INVALID_ARG, "the backward's outputs must not be its inputs");
  }
  const int D = layer->head_dim;
  const int G = layer->num_q_heads / layer->num_kv_heads;
  const int64_t qblocks = ((int64_t)max_seq_len * G + 127) / 128;
  const int64_t kblocks = ((int64_t)max_seq_len + 127) / 128;
  const int64_t pairs = (int64_t)batch * layer->num_kv_heads;
  if (qblocks * pairs > 0x7FFFFFFF || kblocks * pairs * 4 > 0x7FFFFFFF)
    return fail(G4ATTN_ERR_UNSUPPORTED, "grid too large");
  if (batch == 0 || max_seq_len == 0) return ok();
  g4::BackwardArgs a{};
  a.q = q;
  a.k = k;
  a.v = layer->k_eq_v ? k : v;
  a.out = out;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.lse = lse;
  a.delta = delta;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.num_q_heads = layer->num_q_heads;
  a.num_kv_heads = layer->num_kv_heads;
  a.window = layer->window;
  a.num_qblocks = (int32_t)qblocks;
  a.num_kblocks = (int32_t)kblocks;
  a.batch = batch;
  a.scale = layer->softmax_scale;
  a.scale_log2 = (float)((double)layer->softmax_scale * kLog2e);
  const hipError_t e = g4::launch_backward(D, layer->k_eq_v != 0, a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

g4attn_status g4attn_decode(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, const int64_t* cache_row0, const int32_t* ctx_len,
                            int32_t cache_slots, uint16_t* out, int32_t batch, int32_t max_ctx_len,
                            const int32_t* schedule, g4attn_stream_t stream, g4attn_provenance* prov) {
  return decode_impl(layer, q, k_cache, v_cache, cache_row0, ctx_len, cache_slots, out, batch, max_ctx_len, schedule,
                     stream, prov, nullptr);
}

g4attn_status g4attn_split_workspace_bytes(const g4attn_layer* layer, int32_t batch, int32_t rows,
                                           int32_t max_key_len, int32_t split_keys, uint64_t* bytes) {
  if (g4attn_status s = check_layer(layer)) return s;
  if (g4attn_status s = check_split(layer, split_keys)) return s;
  if (!bytes) return fail(G4ATTN_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 0 || rows < 0 || max_key_len < 0)
    return fail(G4ATTN_ERR_INVALID_ARG, "batch, rows and max_key_len must be >= 0");
  *bytes = split_layout(layer, batch, rows, max_key_len, split_keys).bytes;
  return ok();
}

g4attn_status g4attn_prefill_split(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* out, const int32_t* seq_start, const int32_t* seq_len, int32_t batch,
                                   int32_t max_seq_len, int32_t split_keys, void* workspace,
                                   uint64_t workspace_bytes, g4attn_stream_t stream, g4attn_provenance* prov) {
  const SplitRequest sp{split_keys, workspace, workspace_bytes};
  return prefill_impl(layer, q, k, v, out, seq_start, seq_len, nullptr, batch, max_seq_len, stream, prov, &sp);
}

g4attn_status g4attn_prefill_cached_split(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                          const uint16_t* v_cache, uint16_t* out, const int32_t* q_row0,
                                          const int32_t* q_pos0, const int32_t* chunk_len, const int64_t* cache_row0,
                                          int32_t cache_slots, int32_t batch, int32_t max_chunk_len,
                                          int32_t max_key_len, int32_t split_keys, void* workspace,
                                          uint64_t workspace_bytes, g4attn_stream_t stream, g4attn_provenance* prov) {
  const SplitRequest sp{split_keys, workspace, workspace_bytes};
  return cached_impl(layer, q, k_cache, v_cache, out, q_row0, q_pos0, chunk_len, nullptr, cache_row0, cache_slots,
                     batch, max_chunk_len, max_key_len, stream, prov, &sp);
}

g4attn_status g4attn_decode_split(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int64_t* cache_row0, const int32_t* ctx_len,
                                  int32_t cache_slots, uint16_t* out, int32_t batch, int32_t max_ctx_len,
                                  const int32_t* schedule, int32_t split_keys, void* workspace,
                                  uint64_t workspace_bytes, g4attn_stream_t stream, g4attn_provenance* prov) {
  const SplitRequest sp{split_keys, workspace, workspace_bytes};
  return decode_impl(layer, q, k_cache, v_cache, cache_row0, ctx_len, cache_slots, out, batch, max_ctx_len, schedule,
                     stream, prov, &sp);
}

g4attn_status g4attn_decode_split_noalloc(const g4attn_layer* layer, const uint16_t* q, const uint16_t* k_cache,
                                          const uint16_t* v_cache, const int64_t* cache_row0, const int32_t* ctx_len,
                                          int32_t cache_slots, uint16_t* out, int32_t batch, int32_t max_ctx_len,
                                          const int32_t* schedule, int32_t split_keys, g4attn_stream_t stream,
                                          g4attn_provenance* prov) {
  // (the size checks run before the one HIP call that finds the array)
  if (g4attn_status s = check_layer(layer)) return s;
  if (g4attn_status s = check_split(layer, split_keys)) return s;
  if (batch < 0 || max_ctx_len < 0) return fail(G4ATTN_ERR_INVALID_ARG, "batch and max_ctx_len must be >= 0");
  const SplitLayout lay = split_layout(layer, batch, 1, max_ctx_len, split_keys);
  if (lay.bytes > g4::kScratchBytes)
    return fail(G4ATTN_ERR_UNSUPPORTED, "partial results of %llu bytes exceed the library's %llu-byte scratch array "
                "(use g4attn_decode_split with a workspace)", (unsigned long long)lay.bytes,
                (unsigned long long)g4::kScratchBytes);
  void* ws = nullptr;
  if (lay.bytes > 0) {
    const hipError_t e = g4::scratch_address(&ws);
    if (e != hipSuccess) return fail(G4ATTN_ERR_DEVICE, "scratch array lookup failed: %s", hipGetErrorString(e));
  }
  const SplitRequest sp{split_keys, ws, lay.bytes > 0 ? g4::kScratchBytes : 0};
  return decode_impl(layer, q, k_cache, v_cache, cache_row0, ctx_len, cache_slots, out, batch, max_ctx_len, schedule,
                     stream, prov, &sp);
}

}  // extern "C"
