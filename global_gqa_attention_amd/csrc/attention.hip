// attention.hip -- prefill and decode attention kernels for gfx950.
//
// Both kernels run the same tile update (tile.hpp) over KV tiles aligned to position 0
// of their sequence, in ascending order, with no split of the key range: the
// numerical contract of RL-Kernel issue #415 (Gemma-4-31B-it RFC, section 4) asks for
// one fixed reduction order per row and forbids split-KV and cross-work-group atomics.
// Work items covered: sliding_attention_core, global_attention_core (K=V) and the
// decode side of hybrid_kv_cache_contract (same page, section 5).
//
// Work-group: 4 waves x 32 query slots = 128 rows, each row one (position, q head)
// pair of a single KV head; rows are ordered position-major, so the G query heads that
// share a KV head sit next to each other and share every K/V tile read.
// Tiles move global -> LDS with buffer_load ... lds (two stages: the next tile streams
// in while the current one is consumed). Rows outside the sequence, and in decode
// positions outside the visible range, read as zero through the buffer descriptor.
#include <type_traits>

#include "launch.hpp"
#include "tile.hpp"

namespace g4 {

template <int D, bool KEQV>
struct Stage {
  static constexpr int kBytes = Geom<D>::kTileBytes * (KEQV ? 1 : 2);
};

// Runs tiles [t_first, t_last] through the shared tile update. issue(t, lds) starts
// the loads of tile t into the LDS stage at `lds`.
// wq_min / wq_max: the smallest / largest query position of this wave's rows
// (wq_max < 0 when the wave has none); they only decide whether a wave can skip a tile
// that no row of it can see, or skip the mask on a tile that every row sees whole.
// Both shortcuts are exact: a tile without visible keys leaves a row's state unchanged.
template <int D, int DO, bool KEQV, typename Issue>
__device__ __forceinline__ void run_tiles(RowState<DO>& st, lds_char_t* smem, Issue issue,
                                          const bf16x8_t (&qf)[Geom<D>::kKSteps], int t_first, int t_last,
                                          RowBounds rb, int wq_min, int wq_max, int window, float scale_log2,
                                          int slice, int lane) {
  constexpr int kStage = Stage<D, KEQV>::kBytes;
  const LaneOffsets<D> lo = lane_offsets<D>(lane);
  // One tile: returns false when the fast form met a row that must rescale O.
  auto step = [&](int t, int stage, auto rescale_form) -> bool {
    constexpr bool kRescale = decltype(rescale_form)::value;
    const int pos0 = t * kTileKeys;
    const int pos_end = pos0 + kTileKeys - 1;
    const bool any = wq_max >= pos0 && (window == 0 || pos_end > wq_min - window);
    if (!any) return true;
    const bool full = pos_end <= wq_min && (window == 0 || wq_max - pos0 < window);
    const lds_char_t* kt = smem + stage * kStage;
    const lds_char_t* vt = (KEQV ? kt : kt + Geom<D>::kTileBytes) + slice * DO * 2;
    return tile_update<D, DO, kRescale>(st, kt, vt, lo, qf, pos0, rb, scale_log2, !full, lane);
  };
  issue(t_first, smem);
  wait_tile_loads();
  __syncthreads();
  // Fast loop: no O rescale code, so O stays in the accumulator registers.
  int t = t_first;
  bool fast = true;
  for (; t <= t_last; ++t) {
    const int stage = (t - t_first) & 1;
    if (t < t_last) issue(t + 1, smem + (stage ^ 1) * kStage);
    if (!step(t, stage, std::false_type{})) {
      fast = false;
      break;
    }
    wait_tile_loads();
    __syncthreads();
  }
  if (!fast) {
    // Redo tile t with the rescale form from the unchanged state (the load of tile
    // t + 1 was already issued), then continue with the same loads and barriers.
    step(t, (t - t_first) & 1, std::true_type{});
    wait_tile_loads();
    __syncthreads();
    for (++t; t <= t_last; ++t) {
      const int stage = (t - t_first) & 1;
      if (t < t_last) issue(t + 1, smem + (stage ^ 1) * kStage);
      step(t, stage, std::true_type{});
      wait_tile_loads();
      __syncthreads();
    }
  }
}

template <int D, int DO, bool KEQV>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(const PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * Stage<D, KEQV>::kBytes];
  lds_char_t* smem = lds_ptr(smem_raw);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int pairs = Hkv * a.batch;
  // Heaviest query blocks first; the (sequence, KV head) pair varies fastest so that
  // consecutive work-groups (spread over the XCDs) share a query block index.
  constexpr int kSlices = D / DO;  // work-groups that share a query block, one per dim slice
  const int slice = (int)(blockIdx.x % kSlices);
  const unsigned gid = blockIdx.x / kSlices;
  const int pair = (int)(gid % (unsigned)pairs);
  const int qb = a.num_qblocks - 1 - (int)(gid / (unsigned)pairs);
  const int g = pair % Hkv;
  const int b = pair / Hkv;
  const int L = a.seq_len[b];
  const int pos_per_group = kRowsPerGroup / G;
  const int p0 = qb * pos_per_group;
  if (p0 >= L) return;
  const int s0 = a.seq_start[b];

  const int rho = wave * kSlots + (lane & (kSlots - 1));
  const int qp = p0 + rho / G;
  const bool valid = qp < L;
  const int qpos = valid ? qp : -1;
  const int h = g * G + rho % G;
  const int pos_per_wave = kSlots / G;
  const int wq_min = p0 + wave * pos_per_wave;
  const int wq_max = wq_min > L - 1 ? -1 : min(wq_min + pos_per_wave - 1, L - 1);

  bf16x8_t qf[Geom<D>::kKSteps];
  load_q<D>(qf, a.q + ((int64_t)(s0 + (valid ? qp : 0)) * a.num_q_heads + h) * D, valid, lane);
  RowState<DO> st;
  row_state_init<DO>(st);

  // Key rows of this (sequence, KV head) are `stride` bytes apart. Each tile gets a
  // descriptor starting at its first key and ending at the sequence's last key, so the
  // per-lane offsets are loop invariant and keys past the sequence read as zero.
  const uint32_t stride = (uint32_t)Hkv * D * 2;
  const int64_t head0 = ((int64_t)s0 * Hkv + g) * D;
  const uint32_t nrec = (uint32_t)(L - 1) * stride + D * 2;
  const TileLoadMap<D> map = tile_load_map<D>(wave, lane);
  uint32_t voff[TileLoadMap<D>::kInstr];
#pragma unroll
  for (int i = 0; i < TileLoadMap<D>::kInstr; ++i) voff[i] = (uint32_t)map.row[i] * stride + map.chunk_bytes[i];
  const char* kbase = reinterpret_cast<const char*>(a.k + head0);
  const char* vbase = reinterpret_cast<const char*>(a.v + head0);
  auto issue = [&](int t, lds_char_t* lds) {
    const uint32_t shift = (uint32_t)(t * kTileKeys) * stride;
    load_tile<D>(lds, make_rsrc(kbase + shift, nrec - shift), voff, wave);
    if constexpr (!KEQV) load_tile<D>(lds + Geom<D>::kTileBytes, make_rsrc(vbase + shift, nrec - shift), voff, wave);
  };

  const int p_last = min(p0 + pos_per_group - 1, L - 1);
  const int t_first = a.window > 0 ? max(0, p0 - a.window + 1) / kTileKeys : 0;
  const int t_last = p_last / kTileKeys;
  run_tiles<D, DO, KEQV>(st, smem, issue, qf, t_first, t_last, row_bounds(qpos, a.window), wq_min, wq_max,
                         a.window, a.scale_log2, slice, lane);
  if (valid) store_row<DO>(st, a.out + ((int64_t)(s0 + qp) * a.num_q_heads + h) * D + slice * DO, lane);
}

// Decode: one work-group per (sequence, KV head) for the whole head. The query rows are
// the new token's G heads (slots 0..G-1 of a 32-slot score block). Per 64-key tile the
// work of the shared tile update is spread over the waves without changing any row's
// arithmetic: waves 0 and 1 each compute one 32-key score block (the same MFMA chain
// as prefill) and publish its per-row max; every wave forms the same tile max and
// offset; waves 0 and 1 publish P and their per-lane sums; every wave then forms the
// same row sum and accumulates P*V for its own quarter of the head dims, in the same
// block / k-step order as prefill.
// Exchange area of the decode waves (LDS): per-lane floats (block maxima, then block
// sums) at byte 4 l of their array, per-lane P fragments at byte 16 l of theirs.
struct DecodeExchange {
  static constexpr int kMx = 0;                                // float [kBlocks][64]
  static constexpr int kU = kMx + kBlocks * kWave * 4;         // float [kBlocks][64]
  static constexpr int kFloatBytes = kU + kBlocks * kWave * 4;
  static constexpr int kPf = 0;                                // bf16x8 [kBlocks][2][64]
  static constexpr int kPfBytes = kBlocks * 2 * kWave * 16;
  static_assert(kBlocks == 2, "exchange accessors read two blocks");
};

template <int D>
constexpr int decode_chunks_per_wave() {
  return (D / 32) >= kWaves ? (D / 32) / kWaves : 1;
}

template <int D, bool KEQV>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(const DecodeArgs a) {
  constexpr int kStage = Stage<D, KEQV>::kBytes;
  constexpr int NC = decode_chunks_per_wave<D>();
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * kStage];
  __shared__ __attribute__((aligned(16))) char xf_raw[DecodeExchange::kFloatBytes];
  __shared__ __attribute__((aligned(16))) char xp_raw[DecodeExchange::kPfBytes];
  using X = DecodeExchange;
  lds_char_t* smem = lds_ptr(smem_raw);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int g = (int)(blockIdx.x % (unsigned)Hkv);
  const int bs = (int)(blockIdx.x / (unsigned)Hkv);
  const int b = a.schedule ? a.schedule[bs] : bs;
  const int L = a.ctx_len[b];

  const int slot = lane & (kSlots - 1);
  const bool valid = slot < G;
  const int qpos = valid ? L - 1 : -1;
  const int h = g * G + (valid ? slot : 0);
  const RowBounds rb = row_bounds(qpos, a.window);
  const bool scorer = wave < kBlocks;  // waves that compute a score block
  const bool has_chunks = wave * NC < D / 32;

  bf16x8_t qf[Geom<D>::kKSteps];
  load_q<D>(qf, a.q + ((int64_t)b * a.num_q_heads + h) * D, valid && scorer, lane);
  RowState<NC * 32> st;
  row_state_init<NC * 32>(st);
  const LaneOffsets<D> lo = lane_offsets<D>(lane);
  // This lane's slots of the exchange area.
  const uint32_t xf = (uint32_t)(uintptr_t)lds_ptr(xf_raw) + 4 * lane;
  const uint32_t xp = (uint32_t)(uintptr_t)lds_ptr(xp_raw) + 16 * lane;

  const uint32_t stride = (uint32_t)Hkv * D * 2;
  const int64_t head0 = (a.cache_row0[b] * Hkv + g) * D;
  const uint32_t nrec = (uint32_t)a.cache_slots * stride;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_cache + head0, nrec);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_cache + head0, nrec);
  const int first = a.window > 0 ? max(0, L - a.window) : 0;
  const int slots = a.cache_slots;
  const TileLoadMap<D> map = tile_load_map<D>(wave, lane);
  // Cache row of position p: p mod slots, from one scalar modulo per tile.
  auto slot_of = [&](int pos0_mod, int row) -> uint32_t {
    int m = pos0_mod + row;
    if (slots >= kTileKeys) {
      m = m >= slots ? m - slots : m;
    } else {
      m = m % slots;
    }
    return (uint32_t)m;
  };
  // Positions outside [first, L - 1] (not yet written, or overwritten in the ring) read zero.
  auto issue = [&](int t, lds_char_t* lds) {
    const int pos0 = t * kTileKeys;
    const int pos0_mod = pos0 % slots;
    uint32_t voff[TileLoadMap<D>::kInstr];
#pragma unroll
    for (int i = 0; i < TileLoadMap<D>::kInstr; ++i) {
      const int p = pos0 + map.row[i];
      voff[i] = (p >= first && p < L) ? slot_of(pos0_mod, map.row[i]) * stride + map.chunk_bytes[i] : kOutOfRange;
    }
    load_tile<D>(lds, rk, voff, wave);
    if constexpr (!KEQV) load_tile<D>(lds + Geom<D>::kTileBytes, rv, voff, wave);
  };

  const int t_first = first / kTileKeys;
  const int t_last = (L - 1) / kTileKeys;
  issue(t_first, smem);
  wait_tile_loads();
  __syncthreads();
  for (int t = t_first; t <= t_last; ++t) {
    const int stage = (t - t_first) & 1;
    if (t < t_last) issue(t + 1, smem + (stage ^ 1) * kStage);
    const int pos0 = t * kTileKeys;
    const lds_char_t* kt = smem + stage * kStage;
    const lds_char_t* vt = KEQV ? kt : kt + Geom<D>::kTileBytes;
    const bool need_mask = !(pos0 >= first && pos0 + kTileKeys - 1 <= L - 1);
    f32x16_t s[1];
    if (scorer) {
      const uint32_t kb[1] = {(uint32_t)(uintptr_t)kt + wave * kKeyBlock * Geom<D>::kRowBytes};
      score_blocks<D, 1>(s, kb, lo, qf);
      if (need_mask) mask_block(s[0], pos0 + wave * kKeyBlock + 4 * (lane >> 5), rb);
      const float bm = block_max(s[0]);
      if (wave == 0) {
        lds_store_f32<X::kMx>(xf, bm);
      } else {
        lds_store_f32<X::kMx + kWave * 4>(xf, bm);
      }
    }
    exchange_barrier();
    float mx0, mx1;
    lds_load2_f32<X::kMx, X::kMx + kWave * 4>(xf, mx0, mx1);
    float mx = fmaxf(mx0, mx1);
    mx = fmaxf(mx, swap_halves(mx));
    const float tile_max = mx * a.scale_log2;
    float m_new, alpha, offset;
    const bool move = softmax_step(st.m, tile_max, m_new, alpha, offset);
    const bool rescale = __any(move && st.m != kNegInf);
    if (scorer) {
      const float u = exp_block(s[0], a.scale_log2, offset);
      bf16x8_t pw[2];
      pack_p(s[0], pw);
      if (wave == 0) {
        lds_store_b128<X::kPf + 0 * kWave * 16>(xp, pw[0]);
        lds_store_b128<X::kPf + 1 * kWave * 16>(xp, pw[1]);
        lds_store_f32<X::kU>(xf, u);
      } else {
        lds_store_b128<X::kPf + 2 * kWave * 16>(xp, pw[0]);
        lds_store_b128<X::kPf + 3 * kWave * 16>(xp, pw[1]);
        lds_store_f32<X::kU + kWave * 4>(xf, u);
      }
    }
    exchange_barrier();
    float u0, u1;
    lds_load2_f32<X::kU, X::kU + kWave * 4>(xf, u0, u1);
    const float half = u0 + u1;
    const float total = half + swap_halves(half);
    st.l = alpha * st.l + total;
    st.m = m_new;
    if (has_chunks) {
      bf16x8_t pf[kBlocks][2];
      lds_load4_b128<X::kPf, X::kPf + kWave * 16, X::kPf + 2 * kWave * 16, X::kPf + 3 * kWave * 16>(
          xp, pf[0][0], pf[0][1], pf[1][0], pf[1][1]);
      if (rescale) rescale_o<NC * 32>(st, alpha);
      switch (wave) {
        case 0: pv_update<D, NC * 32, 0 * NC>(st, vt, pf, lo); break;
        case 1: if constexpr (1 * NC < D / 32) pv_update<D, NC * 32, 1 * NC>(st, vt, pf, lo); break;
        case 2: if constexpr (2 * NC < D / 32) pv_update<D, NC * 32, 2 * NC>(st, vt, pf, lo); break;
        default: if constexpr (3 * NC < D / 32) pv_update<D, NC * 32, 3 * NC>(st, vt, pf, lo); break;
      }
    }
    wait_tile_loads();
    __syncthreads();
  }
  if (valid && has_chunks) store_row<NC * 32>(st, a.out + ((int64_t)b * a.num_q_heads + h) * D + wave * NC * 32, lane);
}

// Output dims per work-group: the whole head up to 256; a 512-dim head is split over
// two work-groups (each recomputes the same scores and keeps half of O), which keeps
// the O accumulator within the register file.
template <int D>
constexpr int slice_dims() { return D > 256 ? D / 2 : D; }

template <int D, bool KEQV>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  constexpr int DO = slice_dims<D>();
  const unsigned groups = (unsigned)a.num_qblocks * (unsigned)(a.num_kv_heads * a.batch) * (D / DO);
  hipLaunchKernelGGL((prefill_kernel<D, DO, KEQV>), dim3(groups), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool KEQV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const unsigned groups = (unsigned)a.batch * (unsigned)a.num_kv_heads;
  hipLaunchKernelGGL((decode_kernel<D, KEQV>), dim3(groups), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

static void fill_shape(LaunchShape* shape, const char* name) {
  if (!shape) return;
  shape->block_q = kRowsPerGroup;
  shape->block_k = kTileKeys;
  shape->waves = kWaves;
  shape->kernel_name = name;
}

hipError_t launch_prefill(int head_dim, bool k_eq_v, const PrefillArgs& a, hipStream_t stream, LaunchShape* shape) {
#define G4_PREFILL(DD, KV, NAME)                         \
  if (head_dim == DD && k_eq_v == KV) {                  \
    fill_shape(shape, NAME);                             \
    return launch_prefill_t<DD, KV>(a, stream);          \
  }
  G4_PREFILL(64, false, "prefill.d64.kv.mfma32x32x16.bk64")
  G4_PREFILL(64, true, "prefill.d64.keqv.mfma32x32x16.bk64")
  G4_PREFILL(128, false, "prefill.d128.kv.mfma32x32x16.bk64")
  G4_PREFILL(128, true, "prefill.d128.keqv.mfma32x32x16.bk64")
  G4_PREFILL(256, false, "prefill.d256.kv.mfma32x32x16.bk64")
  G4_PREFILL(256, true, "prefill.d256.keqv.mfma32x32x16.bk64")
  G4_PREFILL(512, true, "prefill.d512.keqv.mfma32x32x16.bk64")
#undef G4_PREFILL
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int head_dim, bool k_eq_v, const DecodeArgs& a, hipStream_t stream, LaunchShape* shape) {
#define G4_DECODE(DD, KV, NAME)                          \
  if (head_dim == DD && k_eq_v == KV) {                  \
    fill_shape(shape, NAME);                             \
    return launch_decode_t<DD, KV>(a, stream);           \
  }
  G4_DECODE(64, false, "decode.d64.kv.mfma32x32x16.bk64")
  G4_DECODE(64, true, "decode.d64.keqv.mfma32x32x16.bk64")
  G4_DECODE(128, false, "decode.d128.kv.mfma32x32x16.bk64")
  G4_DECODE(128, true, "decode.d128.keqv.mfma32x32x16.bk64")
  G4_DECODE(256, false, "decode.d256.kv.mfma32x32x16.bk64")
  G4_DECODE(256, true, "decode.d256.keqv.mfma32x32x16.bk64")
  G4_DECODE(512, true, "decode.d512.keqv.mfma32x32x16.bk64")
#undef G4_DECODE
  return hipErrorInvalidValue;
}

}  // namespace g4
