// attention.hip -- prefill and decode attention kernels for gfx950.
//
// Both kernels run the same block update (tile.hpp) over 32-key blocks aligned to
// position 0 of their sequence, in ascending order, with no split of the key range:
// the numerical contract of RL-Kernel issue #415 (Gemma-4-31B-it RFC, section 4) asks
// for one fixed reduction order per row and forbids split-KV and cross-work-group
// atomics. Work items covered: sliding_attention_core, global_attention_core (K=V) and
// the decode side of hybrid_kv_cache_contract (same page, section 5).
#include <algorithm>
#include <atomic>
#include <numeric>
#include <type_traits>

#include "launch.hpp"
#include "tile.hpp"

namespace g4 {

// ===================================================================================
// Prefill
// ===================================================================================
// Work-group: 4 waves x NB N-blocks x 32 query slots, each row one (position, q head)
// pair of a single KV head; rows are ordered position-major, so the G query heads that
// share a KV head sit next to each other and share every K/V block. With NB = 2 a wave
// owns 64 rows and every K/V fragment it reads from LDS feeds two MFMAs, which halves
// the fragment reads and returns per MFMA. The register file holds one wave of these
// tiles per SIMD, and that wave's one instruction stream carries the fragment reads, the
// softmax's vector work and the block loads beside the MFMAs: they, not the matrix cores,
// set the loop's pace.
//
// Each wave runs a software pipeline over the 32-key blocks j of the work-group's key
// range. Iteration j has two scheduling regions: the first holds P*V of block j - 1
// (MFMA) and the softmax of block j (VALU), the second the scores of block j + 1
// (MFMA). Per row the arithmetic is exactly the sequential block update (scores,
// offset step, l, rescale of O, O += P V).
//
// Blocks stream global -> LDS with buffer_load ... lds into NS stages; block j + NS - 1
// is issued at the start of iteration j, into the stage of block j - 1 (whose V was
// last read in iteration j - 1). Keys past the sequence read as zero through the
// buffer descriptor.
// NBW: N-blocks per wave. Two where the 64-row O accumulator fits the register file (the
// default for D <= 256); one for the 512-dim head, and for grids too small to give every
// CU a work-group (twice the work-groups, each half the rows).
// XCDs of the device (MI355X: 8), which receive work-groups in turn.
constexpr int kXcds = 8;

template <int D, bool KEQV, int NBW = (D >= 512 ? 1 : 2)>
struct PrefillCfg {
  // The 512-dim head with separate K and V (64 KiB per block) keeps K and V in rings of
  // their own: kKStages stages of a block's K rows and kVStages of its V rows, 32 KiB each.
  // Every other form keeps one ring of stages, each holding a block's K (and V) rows.
  static constexpr bool kSplit = D >= 512 && !KEQV;
  static constexpr int kKStages = 3;
  static constexpr int kVStages = 2;
  static constexpr int kStageBytes = Geom<D>::kBlockBytes * (KEQV || kSplit ? 1 : 2);
  static constexpr int kStages = 5;  // (split rings: kKStages + kVStages)
  static_assert(!kSplit || kKStages + kVStages == kStages, "split rings fill the stages");
  static constexpr int kLoads = kStageBytes / 1024 / kWaves;  // 1 KiB loads per wave per block
  static constexpr int kNB = NBW;
  static_assert(NBW == 1 || (NBW == 2 && D <= 256), "N-blocks per wave");
  static constexpr int kRows = kRowsPerGroup * kNB;
  // Output staging: a wave's rows in LDS, each padded by 16 bytes.
  static constexpr int kOutRow = Geom<D>::kRowBytes + 16;
  static constexpr int kOutTile = kNB * kSlots * kOutRow;
  // Query rows of the work-group, staged in LDS after stage 0 while the first block loads.
  static constexpr int kQBytes = kRows * Geom<D>::kRowBytes;
  static constexpr int kQLoads = kQBytes / 1024 / kWaves;  // 1 KiB loads per wave
  static constexpr int kSmem = std::max({kStages * kStageBytes, kWaves * kOutTile, kStageBytes + kQBytes});
  static_assert(kLoads >= 1 && kQLoads * 1024 * kWaves == kQBytes && kSmem <= 160 * 1024, "prefill LDS budget");
};

// The passes of a work-group over its key range, each wave owning NB = kNB N-blocks.
// Every key's probability uses its row's final exponent offset (the lazy offset after
// the row's last block; see softmax_step). The first pass takes the offsets as they come:
// for a row whose offset never moves after it holds keys (normalised queries and keys)
// that is already the final offset and the pass's result is the row's result. If some
// row of the work-group did move, the work-group runs the same pass again from the final
// offsets, where no offset moves. Either way no O is ever rescaled, which keeps O in the
// registers the loop accumulates it in.
//
// SPL (the split form of a global layer): the grid repeats over the key chunks (chunk
// slowest), a work-group takes only its chunk's blocks, and a row whose keys span several
// chunks is written as a partial result for the merge; a row whose keys lie in chunk 0
// alone is written whole by the chunk-0 work-group. (In a whole-sequence prefill every
// work-group's rows share their chunks, the chunk size being a multiple of the positions
// of a work-group; chunks of a chunked prefill can start anywhere.)
//
// QP (the q prologue inside the prefill): q holds the raw rows; each wave norms and rotates
// its rows' query fragments as it takes them from LDS, with the q/k prologue's arithmetic in
// its order (so the fragments hold the bits that prologue would have written): the row's
// sum of squares per 8-dim chunk in dim order, then over the chunks as that prologue's
// butterfly adds them (pairs, then quads, ... of chunk indices), 1 / sqrt(mean + eps), the
// weight times the normed value, then the rotation with the angle table of the
// work-group's positions (built in stage 0 before block jf is loaded there).
template <int D, bool KEQV, int NBW, bool LK, bool SPL, bool QP = false>
__device__ __forceinline__ void prefill_pass(const PrefillArgs& a, lds_char_t* smem) {
  using Cfg = PrefillCfg<D, KEQV, NBW>;
  constexpr int NS = Cfg::kStages;
  constexpr int kNB = Cfg::kNB;
  constexpr int NB = kNB;
  constexpr int kStage = Cfg::kStageBytes;
  constexpr int kLoads = Cfg::kLoads;
  constexpr int R = Geom<D>::kRowBytes;
  constexpr bool kSplit = Cfg::kSplit;
  static_assert(!kSplit || NB == 1, "split rings: one N-block per wave");
  // V rows: inside each stage (one ring), or the V ring after the K stages (split rings)
  constexpr int kVOff = KEQV ? 0 : kSplit ? Cfg::kKStages * Cfg::kStageBytes : Geom<D>::kBlockBytes;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int pairs = Hkv * a.batch;
  // Work-groups go to the 8 XCDs in turn (work-group i to XCD i mod 8), each XCD with its
  // own L2. When the (sequence, KV head) pairs split evenly over the XCDs, XCD x takes the
  // query blocks of pair x, then of pair x + 8, ..., each pair's heaviest first: the
  // work-groups an XCD runs together share one pair's K/V (a sliding pair's 4096 keys are
  // 4 MiB, its L2), where the pair-fastest order put four pairs on each L2 at once and
  // fetched their K/V blocks from HBM again. Otherwise: heaviest query blocks first, the
  // pair fastest. (Only the order changes: each row's arithmetic is the same.)
  // (split form: work-group index = chunk x (query blocks x pairs) + the index above; the
  // count per chunk is a multiple of 8 whenever the XCD order applies)
  const unsigned per_chunk = (unsigned)a.num_qblocks * (unsigned)pairs;
  const unsigned gid = SPL ? blockIdx.x % per_chunk : blockIdx.x;
  const int kchunk = SPL ? (int)(blockIdx.x / per_chunk) : 0;
  int pair, qb;
  if (pairs % kXcds == 0) {
    const int x = (int)(gid % (unsigned)kXcds);
    const int k = (int)(gid / (unsigned)kXcds);
    pair = x + kXcds * (k / a.num_qblocks);
    qb = a.num_qblocks - 1 - k % a.num_qblocks;
  } else {
    pair = (int)(gid % (unsigned)pairs);
    qb = a.num_qblocks - 1 - (int)(gid / (unsigned)pairs);
  }
  const int g = pair % Hkv;
  const int b = pair / Hkv;
  // Positions are absolute: the sequence's query rows are positions qpos0 .. L - 1 (rows
  // qrow + qpos0 .. qrow + L - 1 of q and out) and its keys are positions 0 .. L - 1.
  const int nq = a.seq_len[b];
  const int qpos0 = a.q_pos0 ? a.q_pos0[b] : 0;
  const int L = qpos0 + nq;
  const int pos_per_group = Cfg::kRows / G;
  // G is a power of two (the host accepts 1 .. 32): row rho of the work-group is position
  // rho >> lgG, q head g G + (rho & (G - 1)).
  const int lgG = __builtin_ctz((unsigned)G);
  if (qb * pos_per_group >= nq) return;
  const int p0 = qpos0 + qb * pos_per_group;
  const int64_t qrow = (int64_t)a.seq_start[b] - qpos0;
  // (split form: the work-group's rows have keys in chunks 0 .. its last row's / keys)
  const int n_chunks = SPL ? min(p0 + pos_per_group - 1, L - 1) / a.split.keys + 1 : 1;
  if (SPL && kchunk >= n_chunks) return;

  // Rows of the pass's N-block n: slots (wave * kNB + n) * 32 + (l % 32) of the
  // work-group.
  const int pos_per_nblock = kSlots / G;
  int qp[NB], h[NB], nq_min[NB], nq_max[NB];
  bool valid[NB];
  RowBounds rb[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int rho = (wave * kNB + n) * kSlots + (lane & (kSlots - 1));
    qp[n] = p0 + (rho >> lgG);
    valid[n] = qp[n] < L;
    h[n] = g * G + (rho & (G - 1));
    rb[n] = row_bounds(valid[n] ? qp[n] : -1, a.window);
    nq_min[n] = p0 + (wave * kNB + n) * pos_per_nblock;
    nq_max[n] = nq_min[n] > L - 1 ? -1 : min(nq_min[n] + pos_per_nblock - 1, L - 1);
  }
  // Per-row last keys (the rows of an image see every row of that image): a row's key
  // range ends at max(its position, its last key), and the work-group runs the blocks up
  // to the largest of its rows' ends. The test for a block that every row of an N-block
  // sees whole stays the causal one, which is the stricter (a row's end is never below its
  // position), and blocks past a row's end are hidden from it, adding exact zeros.
  int p_end = min(p0 + pos_per_group - 1, L - 1);
  if constexpr (LK) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      if (valid[n]) rb[n].hi = min(max(qp[n], a.last_key[qrow + qp[n]]), L - 1);
    }
    int m = p_end;
    for (int p = p0 + lane; p <= p_end; p += kWave) m = max(m, a.last_key[qrow + p]);
    // (a wait the compiler sees: with none it would wait inside the loop, where its
    // count of loads in flight would also cover the global -> LDS block loads)
    __builtin_amdgcn_s_waitcnt(VmCnt<0>::kImm);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o));
    p_end = __builtin_amdgcn_readfirstlane(min(m, L - 1));
  }
  // Key rows of this (sequence, KV head) are `stride` bytes apart; block j's 32 keys are
  // 32 consecutive rows (position 32 j sits at row 32 j, or at slot 32 j mod slots of a
  // ring whose size is a multiple of 32). Block j's descriptor starts at its first key
  // and ends at the sequence's last key, so the per-lane offsets are loop invariant and
  // keys past the sequence read as zero.
  const uint32_t stride = (uint32_t)Hkv * D * 2;
  const int64_t head0 = ((a.kv_row0 ? a.kv_row0[b] : (int64_t)a.seq_start[b]) * Hkv + g) * D;
  const int slots = a.kv_slots;
  // Load i of this wave fills stage bytes [(wave + 4 i) KiB, +1 KiB): lane l's 16 bytes
  // are the logical chunk that the swizzle puts at that physical position. Within the K
  // (or V) rows of a block, load i covers rows row_a + i * kRowStep (row_a = (wave KiB +
  // 16 lane) / R); the swizzle of a row depends on its low four bits only, so the
  // per-lane part of the offset repeats with period kVPer in i and the rest is the
  // uniform row step. Only the kVPer per-lane parts are kept (behind an empty asm in
  // the loop, so that the compiler does not hoist all kLoads sums into registers).
  constexpr int kRowStep = 4096 / R;
  constexpr int kLoadsPerRegion = Geom<D>::kBlockBytes / 4096 > 0 ? Geom<D>::kBlockBytes / 4096 : 1;
  constexpr int kSwPeriod = 16 / std::gcd(kRowStep, 16);
  constexpr int kVPer = kSwPeriod < kLoadsPerRegion ? kSwPeriod : kLoadsPerRegion;
  uint32_t vo[kVPer];
  {
    const int rbyte = wave * 1024 + lane * 16;  // < 4 KiB <= one region
    const int row_a = rbyte / R;
#pragma unroll
    for (int p = 0; p < kVPer; ++p) {
      const int chunk = ((rbyte % R) >> 4) ^ chunk_swizzle<D>(row_a + p * kRowStep);
      vo[p] = (uint32_t)row_a * stride + (uint32_t)chunk * 16;
    }
  }
  const char* kbase = reinterpret_cast<const char*>(a.k + head0);
  const char* vbase = reinterpret_cast<const char*>(a.v + head0);
  const uint32_t smem0 = lds_addr(smem);
  static_assert(KEQV || Geom<D>::kBlockBytes % (kWaves * 1024) == 0, "K bytes of a block: whole 4 KiB rows");
  // Block j's rows into the stage at LDS byte offset lds_off: its K rows then, in one
  // ring, its V rows; with V_ONLY (split rings) its V rows alone.
  auto issue_at = [&](int j, uint32_t lds_off, auto v_only) {
    constexpr bool kVOnly = decltype(v_only)::value;
    const int pos = j * kBlockKeys;
    const int64_t shift = (int64_t)(slots > 0 ? pos % slots : pos) * stride;
    const uint32_t nrec = (uint32_t)(min(L - pos, kBlockKeys) - 1) * stride + R;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc_uniform((kVOnly ? vbase : kbase) + shift, nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc_uniform(vbase + shift, nrec);
    uint32_t vl[kVPer];
    if constexpr (kSplit) {
      // (the split form has two load sites per iteration and no registers to spare:
      // the per-lane parts are formed afresh from the lane index, which the empty asm
      // keeps the compiler from hoisting)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int rbyte = wave * 1024 + ln * 16;
      const int row_a = rbyte / R;
#pragma unroll
      for (int p = 0; p < kVPer; ++p) {
        const int chunk = ((rbyte % R) >> 4) ^ chunk_swizzle<D>(row_a + p * kRowStep);
        vl[p] = (uint32_t)row_a * stride + (uint32_t)chunk * 16;
      }
    } else {
#pragma unroll
      for (int p = 0; p < kVPer; ++p) {
        vl[p] = vo[p];
        asm volatile("" : "+v"(vl[p]));
      }
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int slot = wave + kWaves * i;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(smem0 + lds_off + (uint32_t)(slot * 1024));
      // (slot KiB >= the K bytes exactly when i does: every wave's slots of load i lie in one
      // 4 KiB row of the stage and the K bytes are a multiple of 4 KiB, so the descriptor is
      // chosen at compile time)
      const bool is_v = !KEQV && !kSplit && i * kWaves * 1024 >= Geom<D>::kBlockBytes;
      const int ii = i % kLoadsPerRegion;
      dma_b128(is_v ? rv : rk, dst, vl[ii % kVPer] + (uint32_t)(ii * kRowStep) * stride);
    }
  };
  auto issue = [&](int j, int stage) { issue_at(j, (uint32_t)(stage * kStage), std::false_type{}); };
  // split rings: K stage s at s * kStage, V stage s after the K stages
  auto issue_v = [&](int j, int stage) {
    issue_at(j, (uint32_t)((Cfg::kKStages + stage) * kStage), std::true_type{});
  };
  // Wait for the block that has `newer` blocks issued after it, then meet the waves.
  auto wait_block = [&](int newer) {
    if (newer >= 3) {
      wait_barrier<3 * kLoads>();
    } else if (newer == 2) {
      wait_barrier<2 * kLoads>();
    } else if (newer == 1) {
      wait_barrier<kLoads>();
    } else {
      wait_barrier<0>();
    }
  };
  auto wrap = [&](int s) { return s >= NS ? s - NS : s; };
  auto wrap_k = [&](int s) { return s >= Cfg::kKStages ? s - Cfg::kKStages : s; };
  auto wrap_v = [&](int s) { return s >= Cfg::kVStages ? s - Cfg::kVStages : s; };

  const int jf = SPL ? kchunk * (a.split.keys / kBlockKeys)
                     : a.window > 0 ? max(0, p0 - a.window + 1) / kBlockKeys : 0;
  const int jl = SPL ? min(p_end, (kchunk + 1) * a.split.keys - 1) / kBlockKeys : p_end / kBlockKeys;
  const float c = a.scale_log2;
  const int kpos_lane = 4 * (lane >> 5);
  // Mask the scores of block j for the N-blocks whose valid rows do not all see it whole.
  auto mask = [&](int j, f32x16_t (&s)[NB]) {
    const int k0 = j * kBlockKeys;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const bool full = k0 + kBlockKeys - 1 <= nq_min[n] && (a.window == 0 || k0 > nq_max[n] - a.window);
      if (!full) mask_block(s[n], k0 + kpos_lane, rb[n]);
    }
  };

  // Prologue: block jf into stage 0 and the query fragments, a wait for both, then
  // blocks jf + 1 .. jf + NS - 2 into stages 1 .. NS - 2 (they land during the first
  // block's work). The wait for everything in flight at that point leaves the compiler
  // no load of its own outstanding inside the loop (its waits there would also stall on
  // the in-flight block loads, which it does not know about).

  // A pass over the key range: iteration j > jf runs [scores of j] then [P*V of j - 1 |
  // softmax of j]. The query fragments are loaded once, before the first pass.
  if constexpr (!QP) issue(jf, 0);
  bf16x8_t qf[NB][Geom<D>::kKSteps];
  {
    // The work-group's query rows come global -> LDS as whole 1 KiB pieces (row rho of
    // the work-group is position p0 + rho / G, q head g G + rho % G; positions at or past
    // the sequence's end read as zero), with their 16-byte chunks swizzled like a K row,
    // into the LDS after stage 0. Each wave then reads its Q^T fragments (16 lanes = 16
    // consecutive rows, one logical chunk: free of bank conflicts), and the stages are
    // released for blocks jf + 1 .. jf + NS - 2.
    const uint32_t qlds = smem0 + kStage;
    {
      constexpr int kPosPerGroup = Cfg::kRows;  // an upper bound of the group's positions (G >= 1)
      const uint32_t qstride = (uint32_t)a.num_q_heads * R;  // bytes between positions
      const int npos = min(L - p0, (kPosPerGroup + G - 1) / G);
      const uint32_t qrec = (uint32_t)(npos - 1) * qstride + (uint32_t)G * R;
      const __amdgpu_buffer_rsrc_t rq =
          make_rsrc_uniform(a.q + ((qrow + p0) * a.num_q_heads + (int64_t)g * G) * D, qrec);
#pragma unroll
      for (int i = 0; i < Cfg::kQLoads; ++i) {
        const int off = (wave + kWaves * i) * 1024 + lane * 16;  // byte of the staged rows
        const int rho = off / R;
        const int chunk = ((off % R) >> 4) ^ chunk_swizzle<D>(rho);
        const uint32_t src = (uint32_t)(rho >> lgG) * qstride + (uint32_t)(rho & (G - 1)) * R + (uint32_t)chunk * 16;
        dma_b128(rq, __builtin_amdgcn_readfirstlane(qlds + (uint32_t)((wave + kWaves * i) * 1024)), src);
      }
    }
    const int half = a.rope_dims >> 1;
    if constexpr (QP) {
      lds_f32_t* cos_t = reinterpret_cast<lds_f32_t*>(smem);
      lds_f32_t* sin_t = cos_t + pos_per_group * half;
      for (int idx = threadIdx.x; idx < pos_per_group * half; idx += kThreads) {
        const int pl = idx / half;
        const int p = p0 + pl;
        float cv = 1.0f, sv = 0.0f;
        if (p < L) rope_cos_sin(a.positions[qrow + p], idx - pl * half, a.rope_theta, a.rope_freq_dim, cv, sv);
        cos_t[idx] = cv;
        sin_t[idx] = sv;
      }
      // q_norm_w after the tables (16-byte aligned): the transform below reads it 16 bytes at a time
      lds_bf16x8_t* wtab = reinterpret_cast<lds_bf16x8_t*>(sin_t + ((pos_per_group * half + 3) & ~3));
      if (threadIdx.x < D / 8) wtab[threadIdx.x] = *reinterpret_cast<const bf16x8_t*>(a.q_norm_w + 8 * threadIdx.x);
      // (the barrier below waits for loads only: the table writes must land before it)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    wait_barrier<0>();
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int rho = (wave * kNB + n) * kSlots + (lane & (kSlots - 1));
      const uint32_t row = qlds + (uint32_t)(rho * R);
      const int sw = chunk_swizzle<D>(rho);
      auto addr = [&](int kk) {
        const int c = 2 * kk + (lane >> 5);
        return row + (uint32_t)((((c & 15) ^ sw) + (c & ~15)) << 4);
      };
      if constexpr (QP) {
        constexpr int KS = Geom<D>::kKSteps;
        auto raw = [&](int kk) { return *reinterpret_cast<const lds_bf16x8_t*>(lds_at(addr(kk))); };
        // sum of squares: per chunk (this lane's 8 dims of k-step kk: chunk 2 kk + l/32) in
        // dim order, the chunk pairs (2 kk, 2 kk + 1) across the lane halves, then the
        // k-steps as a tree over their index bits, low bit first
        float ssq[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const bf16x8_t x = raw(kk);
          float t = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) t = t + (float)x[e] * (float)x[e];
          float lo, hi;
          row_pair(t, lo, hi);
          ssq[kk] = lo + hi;
        }
#pragma unroll
        for (int w = 1; w < KS; w <<= 1) {
#pragma unroll
          for (int kk = 0; kk < KS; kk += 2 * w) ssq[kk] = ssq[kk] + ssq[kk + w];
        }
        const float inv_rms = 1.0f / sqrtf(ssq[0] * (1.0f / (float)D) + a.rms_eps);
        const lds_f32_t* cos_t = reinterpret_cast<const lds_f32_t*>(smem) + (rho >> lgG) * half;
        const lds_f32_t* sin_t = cos_t + pos_per_group * half;
        const lds_bf16x8_t* wtab = reinterpret_cast<const lds_bf16x8_t*>(
            reinterpret_cast<const lds_f32_t*>(smem) + pos_per_group * half + ((pos_per_group * half + 3) & ~3));
        const int po = a.pair_offset / 16;  // the rotation partner's k-step distance
        auto normed = [&](int kk, float (&y)[8]) {
          const bf16x8_t x = raw(kk);
          const bf16x8_t w = wtab[2 * kk + (lane >> 5)];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = (float)w[e] * ((float)x[e] * inv_rms);
        };
        auto put = [&](int kk, const float (&y)[8]) {
          bf16x8_t v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)y[e];
          *reinterpret_cast<lds_bf16x8_t*>(const_cast<lds_char_t*>(lds_at(addr(kk)))) = v;
        };
        // (written back in place, each lane over the chunks it read, a rotated pair
        // together from the raw values; the fragment reads below then take them)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int d0 = 16 * kk + 8 * (lane >> 5);
          const bool first = d0 < half;                                          // with kk + po
          const bool second = d0 >= a.pair_offset && d0 < a.pair_offset + half;  // done with kk - po
          if (second) continue;
          float y[8];
          normed(kk, y);
          if (first) {
            float other[8];
            normed(kk + po, other);
            float ya[8], yb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              ya[e] = y[e] * cos_t[d0 + e] - other[e] * sin_t[d0 + e];
              yb[e] = other[e] * cos_t[d0 + e] + y[e] * sin_t[d0 + e];
            }
            put(kk, ya);
            put(kk + po, yb);
          } else {
            put(kk, y);
          }
        }
      }
      // (straight into the matrix registers, where the score MFMAs read them; four reads
      // in flight, then one wait)
      static_assert(Geom<D>::kKSteps % 4 == 0, "query reads in groups of four");
#pragma unroll
      for (int k4 = 0; k4 < Geom<D>::kKSteps; k4 += 4) {
        u32x4_t w[4];
        asm volatile(
            "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=a"(w[0]), "=a"(w[1]), "=a"(w[2]), "=a"(w[3])
            : "v"(addr(k4)), "v"(addr(k4 + 1)), "v"(addr(k4 + 2)), "v"(addr(k4 + 3)));
#pragma unroll
        for (int u = 0; u < 4; ++u) qf[n][k4 + u] = __builtin_bit_cast(bf16x8_t, w[u]);
      }
    }
    lds_barrier();
  }
  if constexpr (QP) issue(jf, 0);  // (stage 0 held the angle table)
  float m_start[NB];  // each row's offset at the start of a pass
#pragma unroll
  for (int n = 0; n < NB; ++n) m_start[n] = kNegInf;
  for (int pass = 0;; ++pass) {
  if (pass > 0) issue(jf, 0);
  if constexpr (kSplit) {
    // V of block jf, then the K rows of blocks jf + 1 and jf + 2 (V first: the wait before
    // the first iteration then leaves only the newest K block in flight)
    issue_v(jf, 0);
    if (jf + 1 <= jl) issue(jf + 1, 1);
    if (jf + 2 <= jl) issue(jf + 2, 2);
  } else {
#pragma unroll
    for (int t = 1; t < NS - 1; ++t) {
      if (jf + t <= jl) issue(jf + t, t);
    }
  }
  RowState<D> st[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    row_state_init<D>(st[n]);
    st[n].m = m_start[n];
  }
  if constexpr (kSplit) {
    wait_block(1 + min(jl - jf, 2));  // K of block jf (V of jf and up to two K blocks after it)
  } else {
    wait_block(min(jl - jf, NS - 2));
  }
  // ba.k: the K block whose scores are computed next; ba.v: the V block of the next P*V.
  BlockAddr ba;
  {
    const LaneOffsets<D> lo = lane_offsets<D>(lane);
    block_addr_init<D>(ba, lo, smem0, smem0 + kVOff, lane);
  }
  f32x16_t s_cur[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) s_cur[n] = score_block_at<D>(ba, qf[n]);
  bf16x8_t p_cur[NB][2], p_prev[NB][2];
  float alpha[NB];
  // Stage indices of the next score block, the next P*V block and the next load; the
  // stage of block x is (x - jf) mod NS.
  int st_k = 0;
  int st_v = 0;
  int st_ld = NS - 1;
  // (split rings: the K stage and the V stage the next loads go to)
  int st_kld = 0;
  int st_vld = 1;
  // Before the scores of block j + 1 (j < jl): block j + 1 has landed everywhere and,
  // every wave being done with P*V of block j - 1, its stage is free; issue block
  // j + NS - 1 into it. Split rings: K of block j + 1 and V of block j have landed (only
  // K of block j + 2 may still be in flight); V of block j + 1 goes to the V stage of
  // block j - 1 and K of block j + 3 to the K stage of block j, both free.
  auto begin = [&](int j) {
    if constexpr (kSplit) {
      wait_block(j + 2 <= jl ? 1 : 0);
      issue_v(j + 1, st_vld);
      st_vld = wrap_v(st_vld + 1);
      if (j + 3 <= jl) issue(j + 3, st_kld);
      st_kld = wrap_k(st_kld + 1);
      const int nk = wrap_k(st_k + 1);
      block_addr_move(ba, (nk - st_k) * kStage, 0);
      st_k = nk;
    } else {
      wait_block(min(jl, j + NS - 2) - (j + 1));
      if (j + NS - 1 <= jl) issue(j + NS - 1, st_ld);
      st_ld = wrap(st_ld + 1);
      const int nk = wrap(st_k + 1);
      block_addr_move(ba, (nk - st_k) * kStage, 0);
      st_k = nk;
    }
  };
  auto next_v = [&]() {
    const int nv = kSplit ? wrap_v(st_v + 1) : wrap(st_v + 1);
    block_addr_move(ba, 0, (nv - st_v) * kStage);
    st_v = nv;
  };
  bool needed = false;
  if constexpr (NB == 2) {
    // Diagonal placement of the softmax: iteration j runs [scores of j + 1 | softmax of
    // N-block 1 of block j], then [P*V of block j for both N-blocks | softmax of N-block
    // 0 of block j + 1], so each region carries one N-block's softmax. Per row the order
    // of operations is unchanged: offset step, l, then the block's P*V.
    f32x16_t s1_old;
    bf16x8_t p0_next[2];
    mask(jf, s_cur);
    pipelined_step_diag<D, false, false, true, 0>(st, s_cur, p_cur, s_cur[0], p_cur[0], alpha[0], ba, qf, c);
    for (int j = jf; j < jl;) {
      begin(j);
      s1_old = s_cur[1];
      const bool r1 = pipelined_step_diag<D, true, false, true, 1>(st, s_cur, p_cur, s1_old, p_cur[1], alpha[1], ba, qf, c);
      ++j;
      mask(j, s_cur);
      const bool r0 = pipelined_step_diag<D, false, true, true, 0>(st, s_cur, p_cur, s_cur[0], p0_next, alpha[0], ba, qf, c);
      p_cur[0][0] = p0_next[0];
      p_cur[0][1] = p0_next[1];
      next_v();
      needed = needed || r0 || r1;
    }
    // The softmax of N-block 1 of the last block, then its P*V.
    const bool r1 = pipelined_step_diag<D, false, false, true, 1>(st, s_cur, p_cur, s_cur[1], p_cur[1], alpha[1], ba, qf, c);
    needed = needed || r1;
    pipelined_step_diag<D, false, true, false, 0>(st, s_cur, p_cur, s_cur[0], p_cur[0], alpha[0], ba, qf, c);
  } else {
  // Iteration jf: the softmax of jf (the first block cannot need a rescale: every
  // row still has offset -inf).
  mask(jf, s_cur);
  pipelined_step<D, NB, false, true, false>(st, s_cur, s_cur, p_cur, p_cur, alpha, ba, qf, c);
  for (int j = jf; j < jl;) {
    begin(j);
    pipelined_step<D, NB, true, false, false>(st, s_cur, s_cur, p_cur, p_cur, alpha, ba, qf, c);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      p_prev[n][0] = p_cur[n][0];
      p_prev[n][1] = p_cur[n][1];
    }
    ++j;
    mask(j, s_cur);
    const bool resc = pipelined_step<D, NB, false, true, true>(st, s_cur, s_cur, p_cur, p_prev, alpha, ba, qf, c);
    next_v();
    needed = needed || resc;
  }
  // P*V of the last block (split rings: its V rows are the last loads issued).
  if constexpr (kSplit) wait_block(0);
  pipelined_step<D, NB, false, false, true>(st, s_cur, s_cur, p_cur, p_cur, alpha, ba, qf, c);
  }
  // Did some row of the work-group move its offset after it held keys (its O and l then
  // mix two offsets)? A vote through LDS once every wave is done with the stages; if so,
  // the pass runs again from the offsets reached (the second pass moves none).
  lds_barrier();
  if (pass == 0) {
    reinterpret_cast<__attribute__((address_space(3))) int*>(smem)[wave] = needed ? 1 : 0;
    lds_barrier();
    const __attribute__((address_space(3))) int* votes = reinterpret_cast<const __attribute__((address_space(3))) int*>(smem);
    const bool again = (votes[0] | votes[1] | votes[2] | votes[3]) != 0;
    lds_barrier();
    if (again) {
#pragma unroll
      for (int n = 0; n < NB; ++n) m_start[n] = st[n].m;
      continue;
    }
  }
  // Split form, a work-group with rows whose keys span several chunks: each such row's
  // partial result of this chunk (if the row has keys in it), straight from the
  // registers; a row with keys in chunk 0 alone is written whole (the same bits as the
  // tile path below) by the chunk-0 work-group.
  if (SPL && n_chunks > 1) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int nr = qp[n] / a.split.keys + 1;  // the row's chunks
      if (valid[n] && nr == 1 && kchunk == 0) {
        store_row<D>(st[n], a.out + ((qrow + qp[n]) * a.num_q_heads + h[n]) * D, lane);
      } else if (valid[n] && nr > 1 && kchunk < nr) {
        const int64_t part =
            (((int64_t)b * a.split.rows + (qp[n] - qpos0)) * a.num_q_heads + h[n]) * a.split.chunks + kchunk;
        store_partial<D>(st[n], a.split.part_o + part * D, a.split.part_ml + 2 * part, lane);
      }
    }
    break;
  }
  // Output rows out = bf16(O (1 / l)). Each wave puts its rows into its own LDS tile,
  // then writes them back as whole rows, 16 bytes per lane, so that each store
  // instruction covers 1 KiB of contiguous output (two adjacent heads of a position, or
  // one 512-dim row).
  {
    lds_char_t* tile = smem + wave * Cfg::kOutTile;
#pragma unroll
    for (int n = 0; n < NB; ++n) stage_row<D>(st[n], tile + (n * kSlots + (lane & (kSlots - 1))) * Cfg::kOutRow, lane);
    constexpr int kLanesPerRow = R / 16;
    constexpr int kRowsPerStore = kWave / kLanesPerRow;
    const int col = lane % kLanesPerRow;
    // All of the wave's LDS reads first, then the stores (a read sunk into each store's
    // branch would wait out one LDS latency per row).
    constexpr int kStores = NB * kSlots / kRowsPerStore;
    bf16x8_t v[kStores];
#pragma unroll
    for (int i = 0; i < kStores; ++i) {
      const int trow = i * kRowsPerStore + lane / kLanesPerRow;  // n * 32 + slot
      v[i] = *reinterpret_cast<const lds_bf16x8_t*>(tile + trow * Cfg::kOutRow + col * 16);
    }
#pragma unroll
    for (int i = 0; i < kStores; ++i) {
      const int rho = (wave * kNB) * kSlots + i * kRowsPerStore + lane / kLanesPerRow;
      const int qpos = p0 + (rho >> lgG);
      if (qpos < L) {
        *reinterpret_cast<bf16x8_t*>(a.out + ((qrow + qpos) * a.num_q_heads + g * G + (rho & (G - 1))) * D + col * 8) = v[i];
      }
    }
  }
  break;
  }
}

template <int D, bool KEQV, int NBW, bool LK, bool QP = false>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(const PrefillArgs a) {
  using Cfg = PrefillCfg<D, KEQV, NBW>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[Cfg::kSmem];
  prefill_pass<D, KEQV, NBW, LK, false, QP>(a, lds_ptr(smem_raw));
}

// The split form's chunk work-groups (the default N-blocks per wave, causal rows).
template <int D, bool KEQV>
__global__ __launch_bounds__(kThreads, 1) void prefill_split_kernel(const PrefillArgs a) {
  using Cfg = PrefillCfg<D, KEQV>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[Cfg::kSmem];
  prefill_pass<D, KEQV, Cfg::kNB, false, true>(a, lds_ptr(smem_raw));
}

// ===================================================================================
// Decode
// ===================================================================================
// One work-group per (sequence, KV head). The query rows are the new token's G heads
// (slots 0..G-1 of a 32-slot score block). Blocks are taken W at a time (a round; W the
// waves of the work-group): wave w owns block jf + W r + w. Its data (K, and V when
// separate) comes global ->
// registers with 1 KiB contiguous loads one round ahead, and is written to the wave's
// LDS stage at the start of the round. Then, without changing any row's arithmetic:
//   1. wave w computes its block's scores (the same MFMA chain as prefill), masks
//      them, and publishes the row maxima and P and the row sums under the offsets of
//      the round's start;
//   2. if some block of the round moves some row's offset (rare after the first
//      round), every wave steps the row offsets through the round's blocks in order
//      (the same operations as prefill, so the same bits) and wave w recomputes P;
//   3. every wave with output dims updates l block by block and accumulates P*V for
//      its share of the head dims, blocks in order, rescaling O where an offset moved.
// The LDS reads of phases 1 and 3 are inline assembly issued a fixed number of MFMA
// steps ahead, completion tracked with lgkmcnt, as in the prefill loop.
//
// W: waves per work-group. Four, or one (rounds of one block, in a quarter of the LDS, so
// that four work-groups share a CU and one's start and end overlap the others' loads).
template <int D, bool KEQV, int W = kWaves>
struct DecodeCfg {
  // The 512-dim head with separate K and V (64 KiB per block): rounds of two blocks, the K
  // rows of round block b staged by wave b (which computes its scores) and its V rows by
  // wave b + 2. Every other form: rounds of W blocks, wave w staging all of block w.
  static constexpr bool kSplit = D >= 512 && !KEQV;
  static_assert(W == kWaves || (W == 1 && !kSplit), "waves per decode work-group");
  static constexpr int kWavesPG = W;
  static constexpr int kRound = kSplit ? 2 : W;  // blocks per round
  static constexpr int kBlockData = Geom<D>::kBlockBytes * (KEQV || kSplit ? 1 : 2);  // one wave's stage
  static constexpr int kLoads = kBlockData / 1024;  // 1 KiB loads per stage, all by one wave
  static constexpr int kKLoads = kSplit ? kLoads : Geom<D>::kBlockBytes / 1024;  // of which for the first rows
  static constexpr int kLanesPerRow = Geom<D>::kRowBytes / 16;  // 16-byte lanes per key row
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
  static constexpr int kChunks = Geom<D>::kDChunks;
  static constexpr int kNC = kChunks >= W ? kChunks / W : 1;  // output chunks per wave
  static constexpr int kPf = 4;  // MFMA steps the LDS reads run ahead
  static_assert(W * kBlockData + 10 * 1024 <= 160 * 1024, "decode LDS budget");
  static_assert(kBlockData <= 32 * 1024, "stages 0-1 and 2-3 each within a 64 KiB instruction offset");
};

// Wait for this wave's LDS reads; the values are named so no use moves above the wait.
template <int NW>
__device__ __forceinline__ void lds_settle(bf16x8_t (&pw)[NW][2], float (&sw)[NW]) {
#pragma unroll
  for (int w = 0; w < NW; ++w) asm volatile("" : "+v"(pw[w][0]), "+v"(pw[w][1]), "+v"(sw[w]));
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

//
// SPL (the split form, linear caches): the grid repeats over the key chunks (chunk
// slowest, the last chunk index first); a work-group takes its chunk's blocks only, and a
// sequence whose keys span several chunks gets partial results for the merge. (Chunk 0,
// which every sequence has, goes last, so that the launch ends on the short first chunks
// of the short contexts rather than on whole chunks of the long ones: 0.751 -> 0.730 ms
// for 64 contexts in [1024, 32768] at 4096-key chunks.)
template <int D, bool KEQV, bool LIN, bool SPL = false, int W = kWaves>
__global__ __launch_bounds__(W * kWave, 1) void decode_kernel(const DecodeArgs a) {
  using Cfg = DecodeCfg<D, KEQV, W>;
  constexpr int kBlk = Cfg::kBlockData;
  constexpr int NL = Cfg::kLoads;
  constexpr int NKL = Cfg::kKLoads;
  constexpr int NC = Cfg::kNC;
  constexpr int R = Geom<D>::kRowBytes;
  constexpr int KS = Geom<D>::kKSteps;
  constexpr int kPf = Cfg::kPf;
  constexpr bool kSplit = Cfg::kSplit;
  constexpr int BR = Cfg::kRound;
  constexpr int kVOff = KEQV || kSplit ? 0 : Geom<D>::kBlockBytes;  // V rows inside a stage
  __shared__ __attribute__((aligned(1024))) char smem_raw[W * kBlk];
  __shared__ __attribute__((aligned(16))) float xmax[W][kWave];     // block row maxima
  __shared__ __attribute__((aligned(16))) float xsum[W][kWave];     // block row sums of p
  __shared__ __attribute__((aligned(16))) bf16x8_t xp[W][2][kWave];  // P^T fragments
  __shared__ __attribute__((aligned(16))) int xmoved[W];  // block w moves some row's offset
  lds_char_t* smem = lds_ptr(smem_raw);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const unsigned per_chunk = (unsigned)a.batch * (unsigned)Hkv;
  const unsigned gid = SPL ? blockIdx.x % per_chunk : blockIdx.x;
  const int kchunk = SPL ? a.split.chunks - 1 - (int)(blockIdx.x / per_chunk) : 0;
  const int g = (int)(gid % (unsigned)Hkv);
  const int bs = (int)(gid / (unsigned)Hkv);
  const int b = a.schedule ? a.schedule[bs] : bs;
  const int L = a.ctx_len[b];
  // (split form: the row's keys lie in chunks 0 .. (L - 1) / keys)
  const int n_chunks = SPL ? (L - 1) / a.split.keys + 1 : 1;
  if (SPL && kchunk >= n_chunks) return;
  const int key_end = SPL ? min(L, (kchunk + 1) * a.split.keys) : L;  // past the work-group's last key

  const int slot = lane & (kSlots - 1);
  const bool valid = slot < G;
  const int qpos = valid ? L - 1 : -1;
  const int h = g * G + (valid ? slot : 0);
  const RowBounds rb = row_bounds(qpos, a.window);
  // (every wave has output dims unless the head has fewer 32-dim chunks than waves)
  const bool has_chunks = Cfg::kChunks >= W * NC || wave * NC < Cfg::kChunks;

  bf16x8_t qf[KS];
  RowState<NC * 32> st;

  const uint32_t stride = (uint32_t)Hkv * D * 2;
  const int64_t head0 = (a.cache_row0[b] * Hkv + g) * D;
  // A linear cache (no window) holds position p at row p: the descriptor ends after the
  // last visible row, so rows past it (a partial last block, blocks past the last one)
  // read as zero with no per-row test.
  const int vis = min(key_end, a.cache_slots);
  const uint32_t nrec = !LIN ? (uint32_t)a.cache_slots * stride
                             : vis > 0 ? (uint32_t)(vis - 1) * stride + Geom<D>::kRowBytes : 0u;
  // (split rounds: waves 0 .. BR - 1 stage K rows, the others V rows)
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((kSplit && wave >= BR ? a.v_cache : a.k_cache) + head0, nrec);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_cache + head0, nrec);
  const int first = a.window > 0 ? max(0, L - a.window) : 0;
  const int slots = a.cache_slots;
  const int jf = SPL ? kchunk * (a.split.keys / kBlockKeys) : first / kBlockKeys;
  const int jl = (key_end - 1) / kBlockKeys;
  const float c = a.scale_log2;

  // Load i of a block covers bytes [(i % NKL) KiB, +1 KiB) of its K rows (i < NKL) or
  // of its V rows: lane l reads 16 bytes of key row (i % NKL) * kRowsPerLoad + row_a,
  // logical chunk `chunk`.
  const int row_a = lane / Cfg::kLanesPerRow;
  const int chunk = lane % Cfg::kLanesPerRow;
  bf16x8_t buf[NL];
  // Positions outside [first, L - 1] (not yet written, or overwritten in the ring) read
  // as zero; the cache row of position p is p mod slots. A block whose 32 positions are
  // all visible and do not wrap takes the short path: one offset per lane, the row step
  // in the scalar offset.
  // Load i of block j: its lane offset and scalar offset (`interior` and `base` from
  // block_shape).
  auto block_shape = [&](int j, bool& interior, int& base) {
    const int pos0 = j * kBlockKeys;
    base = pos0 % slots;
    interior = pos0 >= first && pos0 + kBlockKeys <= L && base + kBlockKeys <= slots;
  };
  // (One load instruction whatever the path, after the offsets are chosen: with the
  // load outside any branch the compiler counts the loads in flight exactly.)
  auto load_piece = [&](int j, bool interior, int base, int i, bool exists) -> bf16x8_t {
    uint32_t off;
    int soff = 0;
    if (exists && interior) {
      off = (uint32_t)(base + row_a) * stride + (uint32_t)chunk * 16;
      soff = (i % NKL) * Cfg::kRowsPerLoad * (int)stride;
    } else {
      const int row = (i % NKL) * Cfg::kRowsPerLoad + row_a;
      const int p = j * kBlockKeys + row;
      int m = base + row;
      if (slots >= kBlockKeys) {
        m = m >= slots ? m - slots : m;
      } else {
        m = p % slots;
      }
      off = (exists && p >= first && p < L) ? (uint32_t)m * stride + (uint32_t)chunk * 16 : kOutOfRange;
    }
    return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(i < NKL ? rk : rv, (int)off, soff, 0));
  };
  // Block j whole (j <= jl): one branch for the block, the interior path with one lane
  // offset and the row step in the scalar offset.
  auto load_block = [&](int j) {
    bool interior;
    int base;
    block_shape(j, interior, base);
    if (interior) {
      const uint32_t vo = (uint32_t)(base + row_a) * stride + (uint32_t)chunk * 16;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int so = (i % NKL) * Cfg::kRowsPerLoad * (int)stride;
        buf[i] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(i < NKL ? rk : rv, (int)vo, so, 0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) buf[i] = load_piece(j, false, base, i, true);
    }
  };
  // Linear cache: load i of block j at one lane offset per block plus a compile-time row step.
  auto lin_base = [&](int j) -> uint32_t {
    return (uint32_t)(j * kBlockKeys + row_a) * stride + (uint32_t)chunk * 16;
  };
  auto lin_load = [&](uint32_t vb, int i) {
    // (the empty asm keeps the compiler from forming every load's offset at the round's
    // start and holding them all in registers)
    asm volatile("" : "+v"(vb));
    const uint32_t off = vb + (uint32_t)((i % NKL) * Cfg::kRowsPerLoad) * stride;
    buf[i] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(i < NKL ? rk : rv, (int)off, 0, 0));
  };
  lds_char_t* const my_stage = smem + wave * kBlk;
  // The wave's block into its LDS stage, piece by piece, each piece's registers
  // reloaded with the same piece of block jn right after its store: the next round's
  // loads start as this round's data arrives. Loads and stores are unconditional (a
  // block past the last one reads as zero and lands in the wave's own stage, which no
  // wave reads in that round): with no branch around them the compiler counts the loads
  // in flight exactly and waits only for the piece it stores.
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = (i % NKL) * Cfg::kRowsPerLoad + row_a;
      const int region = i / NKL;
      const int phys = chunk ^ chunk_swizzle<D>(row);
      *reinterpret_cast<lds_bf16x8_t*>(my_stage + region * Geom<D>::kBlockBytes + row * R + (phys << 4)) = buf[i];
    }
  };
  auto store_and_load = [&](int jn) {
    bool interior;
    int base;
    block_shape(jn, interior, base);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = (i % NKL) * Cfg::kRowsPerLoad + row_a;
      const int region = i / NKL;
      const int phys = chunk ^ chunk_swizzle<D>(row);
      *reinterpret_cast<lds_bf16x8_t*>(my_stage + region * Geom<D>::kBlockBytes + row * R + (phys << 4)) = buf[i];
      buf[i] = load_piece(jn, interior, base, i, jn <= jl);
    }
  };

  // LDS addresses. Scores: key (l % 32) of the own stage, k-step kk at
  // k_addr[kk % 8] + (kk / 8) * 256 (the swizzled chunk of k-step kk is
  // (2 (kk % 8)) ^ ((l / 32) ^ swizzle(key)) + 16 (kk / 8), the XOR terms sharing no
  // bit). P*V: the transpose reads of output chunk wave * NC + cc, part p, are at
  // v_lo[cc][p] in stages 0 and 1 and v_hi[cc][p] in stages 2 and 3, plus compile-time
  // offsets (stage parity, key step).
  const uint32_t smem0 = lds_addr(smem);
  uint32_t k_addr[8];
  {
    const int key = lane & 31;
    const uint32_t k_row = smem0 + (uint32_t)(wave * kBlk + key * R);
    const uint32_t k_sw = (uint32_t)(((lane >> 5) ^ chunk_swizzle<D>(key)) << 4);
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) k_addr[k8] = k_row + (((uint32_t)k8 << 5) ^ k_sw);
  }
  uint32_t v_lo[NC][2], v_hi[NC][2];
  {
    const int e = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int half = lane & 1;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int cidx = wave * NC + cc;  // output chunk (past the last one for waves without dims: unused)
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const int vkey = 4 * (lane >> 5) + ((lane & 15) >> 2) + 8 * part;
        const int vsw = chunk_swizzle<D>(vkey);
        v_lo[cc][part] = smem0 + (uint32_t)(kVOff + vkey * R + (cidx >> 2) * 256 +
                                            ((((4 * (cidx & 3) + e) ^ vsw) << 4) + (half << 3)));
        v_hi[cc][part] = v_lo[cc][part] + 2 * kBlk;
      }
    }
  }
  auto kread = [&](int kk) -> u32x4_t {
    switch (kk >> 3) {
      case 0: return asm_read_b128_at<0>(k_addr[kk & 7]);
      case 1: return asm_read_b128_at<256>(k_addr[kk & 7]);
      case 2: return asm_read_b128_at<512>(k_addr[kk & 7]);
      default: return asm_read_b128_at<768>(k_addr[kk & 7]);
    }
  };
  // Transpose read pair of P*V step t: block t / (2 NC), chunk (t / 2) % NC, key step t % 2.
  // (split rounds: the V rows of round block w are in stage w + 2)
  constexpr int kSteps = BR * NC * 2;
  auto vread = [&](int t) -> VPair {
    const int w = t / (2 * NC);
    const int cc = (t / 2) % NC;
    const uint32_t b0 = (w < 2 && !kSplit) ? v_lo[cc][0] : v_hi[cc][0];
    const uint32_t b1 = (w < 2 && !kSplit) ? v_lo[cc][1] : v_hi[cc][1];
    switch (((w & 1) << 1) | (t & 1)) {
      case 0: return VPair{asm_read_tr_at<0>(b0), asm_read_tr_at<0>(b1)};
      case 1: return VPair{asm_read_tr_at<16 * R>(b0), asm_read_tr_at<16 * R>(b1)};
      case 2: return VPair{asm_read_tr_at<kBlk>(b0), asm_read_tr_at<kBlk>(b1)};
      default: return VPair{asm_read_tr_at<kBlk + 16 * R>(b0), asm_read_tr_at<kBlk + 16 * R>(b1)};
    }
  };

  const int nrounds = (jl - jf) / BR + 1;
  // Linear caches (K=V: long contexts, hundreds of rounds) pipeline the block loads
  // piece by piece behind the stores; ring caches (a sliding window: a few rounds per
  // sequence) load whole blocks and skip the loads past the last round. The two differ
  // only in when loads are issued, not in what any row computes.
  constexpr bool kPipelined = KEQV || kSplit || LIN;
  // Linear caches issue the next round's loads spread over the scores (the first half)
  // and P*V (the second half), so that the address unit works beside the matrix cores
  // rather than holding up the stores at the round's start.
  constexpr int kH = NL / 2;
  constexpr int kH2 = NL - kH;
  constexpr int kPvSpan = kSteps;  // P*V steps over which the second half is issued
  // Every key's probability uses its row's final exponent offset, as in prefill: the
  // first pass takes the offsets as they come, and if some row moved its offset after it
  // held keys the rounds run again from the final offsets (where none moves).
  float m_start = kNegInf;
  for (int pass = 0;; ++pass) {
  row_state_init<NC * 32>(st);
  st.m = m_start;
  int j_own = jf + wave % BR;
  if constexpr (LIN) {
    const uint32_t vb = lin_base(j_own);
#pragma unroll
    for (int i = 0; i < NL; ++i) lin_load(vb, i);
  } else if constexpr (kPipelined) {
    bool interior;
    int base;
    block_shape(j_own, interior, base);
#pragma unroll
    for (int i = 0; i < NL; ++i) buf[i] = load_piece(j_own, interior, base, i, j_own <= jl);
  } else if (j_own <= jl) {
    load_block(j_own);
  }
  // The query rows load while the first blocks are in flight (one memory latency for
  // both, not two in a row). Then a wait the compiler sees: it then knows the query
  // loads are done and inserts no wait of its own before the score MFMAs inside the loop
  // (where it would also wait for the next round's block loads, which are in flight
  // there).
  if (pass == 0) load_q<D>(qf, a.q + ((int64_t)b * a.num_q_heads + h) * D, valid, lane);
  __builtin_amdgcn_s_waitcnt(VmCnt<0>::kImm);
  bool again = false;
  for (int r = 0; r < nrounds; ++r, j_own += BR) {
    const int nb = min(BR, jl - (jf + BR * r) + 1);  // blocks in this round
    const bool mine = wave < nb;  // this wave computes the scores of round block `wave`
    uint32_t vnext = 0;  // (linear caches) lane offset of the next round's block
    if constexpr (LIN) {
      // Every wave is done with the previous round's LDS; this wave's block (loaded
      // during the previous round) goes to its stage.
      lds_barrier();
      store_block();
      vnext = lin_base(j_own + BR);
    } else if constexpr (kPipelined) {
      // Every wave is done with the previous round's LDS; this wave's block goes to its
      // stage as it arrives, and the next round's block starts loading behind it.
      lds_barrier();
      store_and_load(j_own + BR);
    } else {
      // This wave's block has arrived; every wave is done with the previous round's LDS.
      // (A wave without a block in the last round fills its stage with zeros: the
      // products of its zero probabilities must meet finite values.)
      wait_barrier<0>();
      if (!mine) {
#pragma unroll
        for (int i = 0; i < NL; ++i) buf[i] = bf16x8_t{};
      }
      store_block();
      if (j_own + BR <= jl) load_block(j_own + BR);
    }
    // 1. scores of the own block and their row maxima
    f32x16_t s;
#pragma unroll
    for (int q = 0; q < 16; ++q) s[q] = 0.0f;
    if (mine) {
      u32x4_t kf[kPf + 1];
#pragma unroll
      for (int kk = 0; kk < kPf && kk < KS; ++kk) kf[kk] = kread(kk);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + kPf < KS) kf[(kk + kPf) % (kPf + 1)] = kread(kk + kPf);
        const int after = (kk + kPf < KS ? kk + kPf : KS - 1) - kk;  // reads issued after kk's
        u32x4_t& f = kf[kk % (kPf + 1)];
        if (after >= 4) {
          lds_wait<4>(f);
        } else if (after == 3) {
          lds_wait<3>(f);
        } else if (after == 2) {
          lds_wait<2>(f);
        } else if (after == 1) {
          lds_wait<1>(f);
        } else {
          lds_wait<0>(f);
        }
        s = mfma(as_bf16x8(f), qf[kk], s);
        if constexpr (LIN) {
#pragma unroll
          for (int i = kk * kH / KS; i < (kk + 1) * kH / KS; ++i) lin_load(vnext, i);
        }
      }
      const int k0 = j_own * kBlockKeys;
      if (!(k0 >= first && k0 + kBlockKeys - 1 <= L - 1)) mask_block(s, k0 + 4 * (lane >> 5), rb);
      const float xm = row_max(block_max(s));
      xmax[wave][lane] = xm;
      // (the test of step 2 below, taken here on the wave's own block)
      xmoved[wave] = __any(xm * c > st.m + kRescaleThreshold) ? 1 : 0;
      // The probabilities with the offset of the round's start, which is what every
      // block of the round uses unless one of them moves some row's offset.
      f32x16_t p = s;
      const float u = exp_block(p, c, st.m == kNegInf ? 0.0f : st.m);
      bf16x8_t pf[2];
      pack_p(p, pf);
      xp[wave][0][lane] = pf[0];
      xp[wave][1][lane] = pf[1];
      xsum[wave][lane] = row_sum(u);
    } else {
      // A block past the last one (the last round only): zero probabilities and sums,
      // so that its products add exact zeros and l is unchanged.
      xmoved[wave] = 0;
      xp[wave][0][lane] = bf16x8_t{};
      xp[wave][1][lane] = bf16x8_t{};
      xsum[wave][lane] = 0.0f;
      if constexpr (LIN) {
#pragma unroll
        for (int i = 0; i < kH; ++i) lin_load(vnext, i);
      }
    }
    lds_barrier();
    // 2. Does a block of the round move some row's offset (a block maximum more than the
    // threshold above the row's offset)? Every wave reads the same flags and holds the
    // same offsets, so every wave takes the same branch. If one does, step the offsets
    // through the round's blocks in order (the same operations as prefill) and recompute
    // the probabilities; otherwise every factor is 1. A move after the row held keys
    // sends the work-group to the second pass.
    float alpha[W];
#pragma unroll
    for (int w = 0; w < W; ++w) alpha[w] = 1.0f;
    int moved;
    if constexpr (W == 4) {
      const int4 mvf = *reinterpret_cast<const int4*>(xmoved);  // (one 16-byte read of the flags)
      moved = mvf.x | mvf.y | mvf.z | mvf.w;
    } else {
      moved = xmoved[0];
    }
    if (__builtin_amdgcn_readfirstlane(moved) != 0) {
      float tmax[W];
#pragma unroll
      for (int w = 0; w < W; ++w) tmax[w] = w < nb ? xmax[w][lane] * c : kNegInf;
      float off_own = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        if (w < nb) {
          float m_new, offset;
          const bool move = softmax_step(st.m, tmax[w], m_new, alpha[w], offset);
          again = again || __any(move && st.m != kNegInf);
          if (w == wave) off_own = offset;
          st.m = m_new;
        }
      }
      // (no wave reads P before the next barrier)
      if (mine) {
        const float u = exp_block(s, c, off_own);
        bf16x8_t pf[2];
        pack_p(s, pf);
        xp[wave][0][lane] = pf[0];
        xp[wave][1][lane] = pf[1];
        xsum[wave][lane] = row_sum(u);
      }
      lds_barrier();
    }
    // 3. l and this wave's share of O, block by block (reads run kPf steps ahead; the
    // first V reads go out before those of P, so that one wait covers both)
    if (has_chunks) {
      VPair vf[kPf + 1];
#pragma unroll
      for (int t = 0; t < kPf; ++t) vf[t] = vread(t);
      bf16x8_t pw[W][2];
      float sw[W];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        pw[w][0] = xp[w][0][lane];
        pw[w][1] = xp[w][1][lane];
        sw[w] = xsum[w][lane];
      }
      lds_settle<W>(pw, sw);
      // (no test around a product: the last round's absent blocks have zero
      // probabilities, and a test would make the compiler copy the accumulators at every
      // step)
#pragma unroll
      for (int t = 0; t < kSteps; ++t) {
        const int w = t / (2 * NC);
        const int cc = (t / 2) % NC;
        if (t + kPf < kSteps) vf[(t + kPf) % (kPf + 1)] = vread(t + kPf);
        const int after = 2 * ((t + kPf < kSteps ? t + kPf : kSteps - 1) - t);  // reads issued after t's
        VPair& f = vf[t % (kPf + 1)];
        if (after >= 8) {
          lds_wait<8>(f);
        } else if (after == 6) {
          lds_wait<6>(f);
        } else if (after == 4) {
          lds_wait<4>(f);
        } else if (after == 2) {
          lds_wait<2>(f);
        } else {
          lds_wait<0>(f);
        }
        if (t % (2 * NC) == 0) st.l = alpha[w] * st.l + sw[w];
        st.o[cc] = mfma(as_bf16x8(f), pw[w][t & 1], st.o[cc]);
        if constexpr (LIN) {
          if (t < kPvSpan) {
#pragma unroll
            for (int i = kH + t * kH2 / kPvSpan; i < kH + (t + 1) * kH2 / kPvSpan; ++i) lin_load(vnext, i);
          }
        }
      }
    } else if constexpr (LIN) {
#pragma unroll
      for (int i = kH; i < NL; ++i) lin_load(vnext, i);
    }
  }
  if (pass == 0 && again) {
    m_start = st.m;
    continue;
  }
  if (SPL && n_chunks > 1) {
    // the chunk's partial result (wave 0 also writes the row's offset and sum)
    if (valid && has_chunks) {
      const int64_t part = (((int64_t)b * a.split.rows) * a.num_q_heads + h) * a.split.chunks + kchunk;
      store_partial<NC * 32>(st, a.split.part_o + part * D + wave * NC * 32,
                             wave == 0 ? a.split.part_ml + 2 * part : nullptr, lane);
    }
  } else if (valid && has_chunks) {
    store_row<NC * 32>(st, a.out + ((int64_t)b * a.num_q_heads + h) * D + wave * NC * 32, lane);
  }
  break;
  }
}


// ===================================================================================
// Merge of the split form
// ===================================================================================
// One wave per row with keys in n >= 2 chunks: M = the largest chunk offset; then, the
// chunks in ascending order, w_c = 2^(m_c - M), L = w_0 l_0 + w_1 l_1 + ... and
// O = w_0 O_0 + w_1 O_1 + ... (fp32, left to right, a product then a sum at each step);
// out = bf16(O (1 / L)). Prefill and decode rows go through this one function, so equal
// partials give equal outputs. Lane l takes dims E l .. E l + E - 1 (E = D / 64).
template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeArgs a) {
  constexpr int E = D / kWave;
  typedef float fE_t __attribute__((ext_vector_type(E)));
  typedef __bf16 bE_t __attribute__((ext_vector_type(E)));
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  const int Hq = a.num_q_heads;
  const int h = (int)(r % Hq);
  const int span = a.rows - a.row_skip;  // rows per sequence in the grid
  const int64_t bs = r / Hq;
  const int i = (int)(bs % span) + a.row_skip;
  const int b = (int)(bs / span);
  const int64_t bi = (int64_t)b * a.rows + i;  // the row's slot in the partial layout
  if (b >= a.batch || i >= (a.nrows ? a.nrows[b] : 1)) return;
  const int pos = (a.pos_ref ? a.pos_ref[b] : 0) + a.pos_bias + i;
  const int n = pos / a.split_keys + 1;
  if (n < 2) return;
  const int64_t p0 = (bi * Hq + h) * a.chunks;  // the row's partial of chunk 0
  float M = kNegInf;
  for (int c = 0; c < n; ++c) M = fmaxf(M, a.part_ml[2 * (p0 + c)]);
  fE_t o;
  float l = 0.0f;
  for (int c = 0; c < n; ++c) {
    const float w = exp2_hw(a.part_ml[2 * (p0 + c)] - M);
    const float lc = a.part_ml[2 * (p0 + c) + 1];
    const fE_t v = *reinterpret_cast<const fE_t*>(a.part_o + (p0 + c) * D + E * lane);
    if (c == 0) {
      l = w * lc;
      o = w * v;
    } else {
      l = l + w * lc;
      o = o + w * v;
    }
  }
  const float inv = 1.0f / l;
  bE_t y;
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = (__bf16)(o[e] * inv);
  const int64_t orow = (a.out_row0 ? (int64_t)a.out_row0[b] : (int64_t)b) + i;
  *reinterpret_cast<bE_t*>(a.out + (orow * Hq + h) * D + E * lane) = y;
}

// ===================================================================================
// The library's scratch array
// ===================================================================================
// Partial results of the split form for callers that pass no workspace. In host code the
// array's name stands for no device address: kernels get the address that
// hipGetSymbolAddress returns for the current device (each GPU holds its own copy).
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxScratchDevices];

hipError_t scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

// ===================================================================================
// Launchers
// ===================================================================================
template <int D, bool KEQV, int NBW, bool LK = false>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  const unsigned groups = (unsigned)a.num_qblocks * (unsigned)(a.num_kv_heads * a.batch);
  hipLaunchKernelGGL((prefill_kernel<D, KEQV, NBW, LK>), dim3(groups), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// A sliding window gives every (sequence, KV head) the same few rounds: one-wave
// work-groups (head dims up to 256) in a quarter of the LDS, four per CU, so that one's
// first loads and last round overlap the others' streaming (each CU still runs one wave
// per SIMD; 64 sequences
// of a 1024-key window: 0.200 ms in four-wave work-groups, 0.184 in two-wave ones, 0.180
// in one-wave ones). Linear caches
// (whole contexts, up to hundreds of rounds for the longest sequences, which bound the
// launch) keep four waves per work-group: a sequence streams through one CU, and four
// waves keep more of it in flight.
template <int D, bool KEQV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream, LaunchShape* shape) {
  const unsigned groups = (unsigned)a.batch * (unsigned)a.num_kv_heads;
  if (a.window == 0) {
    hipLaunchKernelGGL((decode_kernel<D, KEQV, true>), dim3(groups), dim3(kThreads), 0, stream, a);
  } else {
    constexpr int W = D >= 512 ? kWaves : 1;  // (one wave would hold all 512 dims of O)
    if (shape) shape->waves = W;
    hipLaunchKernelGGL((decode_kernel<D, KEQV, false, false, W>), dim3(groups), dim3(W * kWave), 0, stream, a);
  }
  return hipGetLastError();
}

int prefill_rows_per_group(int head_dim, bool k_eq_v, bool narrow) {
  if (head_dim >= 512 || narrow) return kRowsPerGroup;
  return 2 * kRowsPerGroup;
}

static void fill_shape(LaunchShape* shape, const char* name, int block_q = kRowsPerGroup) {
  if (!shape) return;
  shape->block_q = block_q;
  shape->block_k = kBlockKeys;
  shape->waves = kWaves;
  shape->kernel_name = name;
}

// The prefill with the q prologue inside (head dim 512, one tensor as K and V).
hipError_t launch_prefill_qp(const PrefillArgs& a, hipStream_t stream, LaunchShape* shape) {
  fill_shape(shape, "prefill.d512.keqv.mfma32x32x16.bk32.qprologue", PrefillCfg<512, true>::kRows);
  const unsigned groups = (unsigned)a.num_qblocks * (unsigned)(a.num_kv_heads * a.batch);
  hipLaunchKernelGGL((prefill_kernel<512, true, 1, false, true>), dim3(groups), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill(int head_dim, bool k_eq_v, bool narrow, const PrefillArgs& a, hipStream_t stream,
                          LaunchShape* shape) {
  const bool last_key = a.last_key != nullptr;
#define G4_PREFILL(DD, KV, NAME)                                                         \
  if (head_dim == DD && k_eq_v == KV) {                                                  \
    if (DD < 512 && narrow) {                                                            \
      fill_shape(shape, last_key ? NAME ".nb1.lastkey" : NAME ".nb1", PrefillCfg<DD, KV, 1>::kRows); \
      return last_key ? launch_prefill_t<DD, KV, 1, true>(a, stream) : launch_prefill_t<DD, KV, 1>(a, stream); \
    }                                                                                    \
    fill_shape(shape, last_key ? NAME ".lastkey" : NAME, PrefillCfg<DD, KV>::kRows);    \
    return last_key ? launch_prefill_t<DD, KV, PrefillCfg<DD, KV>::kNB, true>(a, stream) \
                    : launch_prefill_t<DD, KV, PrefillCfg<DD, KV>::kNB>(a, stream);      \
  }
  G4_PREFILL(64, false, "prefill.d64.kv.mfma32x32x16.bk32")
  G4_PREFILL(64, true, "prefill.d64.keqv.mfma32x32x16.bk32")
  G4_PREFILL(128, false, "prefill.d128.kv.mfma32x32x16.bk32")
  G4_PREFILL(128, true, "prefill.d128.keqv.mfma32x32x16.bk32")
  G4_PREFILL(256, false, "prefill.d256.kv.mfma32x32x16.bk32")
  G4_PREFILL(256, true, "prefill.d256.keqv.mfma32x32x16.bk32")
  G4_PREFILL(512, true, "prefill.d512.keqv.mfma32x32x16.bk32")
  G4_PREFILL(512, false, "prefill.d512.kv.mfma32x32x16.bk32")
#undef G4_PREFILL
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_merge_t(const MergeArgs& m, hipStream_t stream) {
  const int64_t rows = (int64_t)m.batch * (m.rows - m.row_skip) * m.num_q_heads;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kThreads), 0, stream, m);
  return hipGetLastError();
}

static hipError_t launch_merge(int head_dim, const MergeArgs& m, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_merge_t<64>(m, stream);
    case 128: return launch_merge_t<128>(m, stream);
    case 256: return launch_merge_t<256>(m, stream);
    case 512: return launch_merge_t<512>(m, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_split(int head_dim, bool k_eq_v, const PrefillArgs& a, const MergeArgs& m,
                                hipStream_t stream, LaunchShape* shape) {
  const unsigned groups =
      (unsigned)a.num_qblocks * (unsigned)(a.num_kv_heads * a.batch) * (unsigned)a.split.chunks;
  hipError_t e = hipErrorInvalidValue;
#define G4_PREFILL_SPLIT(DD, KV, NAME)                                                                   \
  if (head_dim == DD && k_eq_v == KV) {                                                                  \
    fill_shape(shape, NAME, PrefillCfg<DD, KV>::kRows);                                                  \
    hipLaunchKernelGGL((prefill_split_kernel<DD, KV>), dim3(groups), dim3(kThreads), 0, stream, a);     \
    e = hipGetLastError();                                                                               \
  }
  G4_PREFILL_SPLIT(64, false, "prefill.d64.kv.mfma32x32x16.bk32.split")
  G4_PREFILL_SPLIT(64, true, "prefill.d64.keqv.mfma32x32x16.bk32.split")
  G4_PREFILL_SPLIT(128, false, "prefill.d128.kv.mfma32x32x16.bk32.split")
  G4_PREFILL_SPLIT(128, true, "prefill.d128.keqv.mfma32x32x16.bk32.split")
  G4_PREFILL_SPLIT(256, false, "prefill.d256.kv.mfma32x32x16.bk32.split")
  G4_PREFILL_SPLIT(256, true, "prefill.d256.keqv.mfma32x32x16.bk32.split")
  G4_PREFILL_SPLIT(512, true, "prefill.d512.keqv.mfma32x32x16.bk32.split")
  G4_PREFILL_SPLIT(512, false, "prefill.d512.kv.mfma32x32x16.bk32.split")
#undef G4_PREFILL_SPLIT
  if (e != hipSuccess) return e;
  return launch_merge(head_dim, m, stream);
}

hipError_t launch_decode_split(int head_dim, bool k_eq_v, const DecodeArgs& a, const MergeArgs& m,
                               hipStream_t stream, LaunchShape* shape) {
  const unsigned groups = (unsigned)a.batch * (unsigned)a.num_kv_heads * (unsigned)a.split.chunks;
  hipError_t e = hipErrorInvalidValue;
#define G4_DECODE_SPLIT(DD, KV, NAME)                                                                   \
  if (head_dim == DD && k_eq_v == KV) {                                                                 \
    fill_shape(shape, NAME);                                                                            \
    hipLaunchKernelGGL((decode_kernel<DD, KV, true, true>), dim3(groups), dim3(kThreads), 0, stream, a);     \
    e = hipGetLastError();                                                                              \
  }
  G4_DECODE_SPLIT(64, false, "decode.d64.kv.mfma32x32x16.bk32.split")
  G4_DECODE_SPLIT(64, true, "decode.d64.keqv.mfma32x32x16.bk32.split")
  G4_DECODE_SPLIT(128, false, "decode.d128.kv.mfma32x32x16.bk32.split")
  G4_DECODE_SPLIT(128, true, "decode.d128.keqv.mfma32x32x16.bk32.split")
  G4_DECODE_SPLIT(256, false, "decode.d256.kv.mfma32x32x16.bk32.split")
  G4_DECODE_SPLIT(256, true, "decode.d256.keqv.mfma32x32x16.bk32.split")
  G4_DECODE_SPLIT(512, true, "decode.d512.keqv.mfma32x32x16.bk32.split")
  G4_DECODE_SPLIT(512, false, "decode.d512.kv.mfma32x32x16.bk32.split")
#undef G4_DECODE_SPLIT
  if (e != hipSuccess) return e;
  return launch_merge(head_dim, m, stream);
}

hipError_t launch_decode(int head_dim, bool k_eq_v, const DecodeArgs& a, hipStream_t stream, LaunchShape* shape) {
#define G4_DECODE(DD, KV, NAME)                       \
  if (head_dim == DD && k_eq_v == KV) {               \
    fill_shape(shape, NAME);                          \
    return launch_decode_t<DD, KV>(a, stream, shape); \
  }
  G4_DECODE(64, false, "decode.d64.kv.mfma32x32x16.bk32")
  G4_DECODE(64, true, "decode.d64.keqv.mfma32x32x16.bk32")
  G4_DECODE(128, false, "decode.d128.kv.mfma32x32x16.bk32")
  G4_DECODE(128, true, "decode.d128.keqv.mfma32x32x16.bk32")
  G4_DECODE(256, false, "decode.d256.kv.mfma32x32x16.bk32")
  G4_DECODE(256, true, "decode.d256.keqv.mfma32x32x16.bk32")
  G4_DECODE(512, true, "decode.d512.keqv.mfma32x32x16.bk32")
  G4_DECODE(512, false, "decode.d512.kv.mfma32x32x16.bk32")
#undef G4_DECODE
  return hipErrorInvalidValue;
}

}  // namespace g4
